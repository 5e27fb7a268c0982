// k_ceiling.hip -- measurement kernels for the HBM ceilings of the traffic
// patterns the Atom kernels move: pure streaming reads, pure streaming
// writes, a copy, and a 1 -> P fan-out (one load, P stores), the last also
// with the P stores issued in a rotated order and as pure writes to P
// buffers (no load). Built into a library of its own, libatom_ceiling.so,
// used only by the benchmark's ceiling mode; no collective runs here.
//
// Each kernel moves tiles of lanes * U 16-byte slots, one tile per
// workgroup (the launch shape of the zero-staging Atom kernels); reads are
// non-temporal loads, writes non-temporal buffer stores. Every entry point
// checks its sizes on the host: bytes must be a positive multiple of 16 and
// every buffer 16-byte aligned.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "atom_dev.hpp"

namespace atom {
namespace {

constexpr int kMaxFan = 16;

struct FanArgs {
    char* dst[kMaxFan];
    const char* src;
    int64_t n16;        // 16-byte slots per stream
    int64_t block_tiles;  // blocked order: tiles per block
    int32_t ndst;
    int32_t rotate;     // 1: tile t stores to outputs (t + i) mod ndst, i = 0..ndst-1
    int32_t cached;     // blocked order: 1 = ordinary loads (kept in the caches), 0 = streaming
};

template <int U>
__global__ __launch_bounds__(256) void k_fill(char* d, int64_t n16)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * blockDim.x * U;
    const u32x4 v = {1u, 2u, 3u, static_cast<uint32_t>(blockIdx.x)};
    char* tile = d + base * kVecBytes;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + u * blockDim.x + threadIdx.x;
        if (i < n16)
            st16(tile, static_cast<uint32_t>(u * blockDim.x + threadIdx.x) * kVecBytes, v, true);
    }
}

template <int U>
__global__ __launch_bounds__(256) void k_read(const char* s, int64_t n16, uint32_t* sink)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * blockDim.x * U;
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + u * blockDim.x + threadIdx.x;
        x[u] = i < n16 ? ld16_stream(s + i * kVecBytes) : u32x4{0, 0, 0, 0};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
        acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
    if (acc == 0x9E3779B9u)     // practically never true; keeps the loads
        sink[0] = acc;
}

template <int U>
__global__ __launch_bounds__(256) void k_fan(const FanArgs a)
{
    const int64_t base = static_cast<int64_t>(blockIdx.x) * blockDim.x * U;
    u32x4 x[U];
    if (a.src) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * blockDim.x + threadIdx.x;
            if (i < a.n16)
                x[u] = ld16_stream(a.src + i * kVecBytes);
        }
    } else {                     // pure writes: a constant per tile
#pragma unroll
        for (int u = 0; u < U; ++u)
            x[u] = u32x4{1u, 2u, 3u, static_cast<uint32_t>(blockIdx.x)};
    }
    for (int k = 0; k < a.ndst; ++k) {
        int q = k;
        if (a.rotate) {
            q = static_cast<int>((blockIdx.x + k) % a.ndst);
        }
        char* tile = a.dst[q] + base * kVecBytes;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * blockDim.x + threadIdx.x;
            if (i < a.n16)
                st16(tile, static_cast<uint32_t>(u * blockDim.x + threadIdx.x) * kVecBytes, x[u], true);
        }
    }
}

// Blocked order: the tiles are cut into blocks of block_tiles; workgroups
// take (block, output, tile) in that nesting, so the chip writes one output
// at a time, block by block, and each source tile is loaded once per output
// (after the first, from the caches when `cached`).
template <int U>
__global__ __launch_bounds__(256) void k_fan_blocked(const FanArgs a)
{
    const int64_t tile_slots = static_cast<int64_t>(blockDim.x) * U;
    const int64_t ntiles = (a.n16 + tile_slots - 1) / tile_slots;
    const int64_t per_block = a.block_tiles * a.ndst;
    const int64_t w = blockIdx.x;
    const int64_t b = w / per_block, rem = w - b * per_block;
    const int q = static_cast<int>(rem / a.block_tiles);
    const int64_t t = b * a.block_tiles + (rem - static_cast<int64_t>(q) * a.block_tiles);
    if (t >= ntiles)
        return;
    const int64_t base = t * tile_slots;
    // The load policy is an immediate of each branch's buffer load, so the
    // compiler cannot merge the two loads into one and drop the hint.
    const auto rs = stream_rsrc(a.src + base * kVecBytes, static_cast<uint32_t>(tile_slots * kVecBytes));
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + u * blockDim.x + threadIdx.x;
        const int off = static_cast<int>((u * blockDim.x + threadIdx.x) * kVecBytes);
        if (i < a.n16) {
            if (a.cached)
                x[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
            else
                x[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCpolNt);
        }
    }
    char* tile = a.dst[q] + base * kVecBytes;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + u * blockDim.x + threadIdx.x;
        if (i < a.n16)
            st16(tile, static_cast<uint32_t>(u * blockDim.x + threadIdx.x) * kVecBytes, x[u], true);
    }
}

bool ok16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && p != nullptr; }

bool shape_ok(int64_t bytes, int lanes, int U)
{
    return bytes > 0 && bytes % 16 == 0 && (lanes == 64 || lanes == 128 || lanes == 256) &&
           (U == 1 || U == 2 || U == 4);
}

int64_t grid_of(int64_t n16, int lanes, int U) { return (n16 + lanes * U - 1) / (lanes * U); }

int status(hipError_t e) { return e == hipSuccess ? 0 : 3; }

}  // namespace
}  // namespace atom

using namespace atom;

extern "C" {

// Streaming write of `bytes` bytes. Returns 0, 1 (bad argument) or 3 (HIP).
int ceil_fill(void* dst, int64_t bytes, int lanes, int U, void* stream)
{
    if (!ok16(dst) || !shape_ok(bytes, lanes, U))
        return 1;
    const int64_t n16 = bytes / 16, g = grid_of(n16, lanes, U);
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* d = static_cast<char*>(dst);
    switch (U) {
    case 1: k_fill<1><<<g, lanes, 0, s>>>(d, n16); break;
    case 2: k_fill<2><<<g, lanes, 0, s>>>(d, n16); break;
    default: k_fill<4><<<g, lanes, 0, s>>>(d, n16); break;
    }
    return status(hipGetLastError());
}

// Streaming read of `bytes` bytes; `sink` is 4 device bytes (never
// written in practice).
int ceil_read(const void* src, int64_t bytes, void* sink, int lanes, int U, void* stream)
{
    if (!ok16(src) || !ok16(sink) || !shape_ok(bytes, lanes, U))
        return 1;
    const int64_t n16 = bytes / 16, g = grid_of(n16, lanes, U);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const char* p = static_cast<const char*>(src);
    uint32_t* k = static_cast<uint32_t*>(sink);
    switch (U) {
    case 1: k_read<1><<<g, lanes, 0, s>>>(p, n16, k); break;
    case 2: k_read<2><<<g, lanes, 0, s>>>(p, n16, k); break;
    default: k_read<4><<<g, lanes, 0, s>>>(p, n16, k); break;
    }
    return status(hipGetLastError());
}

// The 1 -> ndst fan-out in blocked order (k_fan_blocked): blocks of
// block_bytes (a multiple of the tile), cached = ordinary source loads.
int ceil_fanout_blocked(void* const* dsts, int ndst, const void* src, int64_t bytes,
                        int64_t block_bytes, int cached, int lanes, int U, void* stream)
{
    if (!dsts || ndst < 1 || ndst > kMaxFan || !ok16(src) || !shape_ok(bytes, lanes, U))
        return 1;
    const int64_t tile_bytes = static_cast<int64_t>(lanes) * U * 16;
    if (block_bytes < tile_bytes || block_bytes % tile_bytes)
        return 1;
    FanArgs a{};
    for (int q = 0; q < ndst; ++q) {
        if (!ok16(dsts[q]))
            return 1;
        a.dst[q] = static_cast<char*>(dsts[q]);
    }
    a.src = static_cast<const char*>(src);
    a.n16 = bytes / 16;
    a.ndst = ndst;
    a.block_tiles = block_bytes / tile_bytes;
    a.cached = cached ? 1 : 0;
    const int64_t ntiles = (a.n16 + lanes * U - 1) / (lanes * U);
    const int64_t nblocks = (ntiles + a.block_tiles - 1) / a.block_tiles;
    const int64_t g = nblocks * a.block_tiles * ndst;
    if (g > 0x7FFFFFFF)
        return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (U) {
    case 1: k_fan_blocked<1><<<g, lanes, 0, s>>>(a); break;
    case 2: k_fan_blocked<2><<<g, lanes, 0, s>>>(a); break;
    default: k_fan_blocked<4><<<g, lanes, 0, s>>>(a); break;
    }
    return status(hipGetLastError());
}

// `bytes` of src to each of ndst (1..16) destinations; src == NULL writes
// a constant instead (pure writes). rotate: tile t stores to its outputs
// starting at t mod ndst. A copy is ndst = 1.
int ceil_fanout(void* const* dsts, int ndst, const void* src, int64_t bytes, int rotate,
                int lanes, int U, void* stream)
{
    if (!dsts || ndst < 1 || ndst > kMaxFan || (src && !ok16(src)) || !shape_ok(bytes, lanes, U))
        return 1;
    FanArgs a{};
    for (int q = 0; q < ndst; ++q) {
        if (!ok16(dsts[q]))
            return 1;
        a.dst[q] = static_cast<char*>(dsts[q]);
    }
    a.src = static_cast<const char*>(src);
    a.n16 = bytes / 16;
    a.ndst = ndst;
    a.rotate = rotate ? 1 : 0;
    const int64_t g = grid_of(a.n16, lanes, U);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (U) {
    case 1: k_fan<1><<<g, lanes, 0, s>>>(a); break;
    case 2: k_fan<2><<<g, lanes, 0, s>>>(a); break;
    default: k_fan<4><<<g, lanes, 0, s>>>(a); break;
    }
    return status(hipGetLastError());
}

}  // extern "C"
