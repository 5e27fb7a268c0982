// k_reduce.hip -- the Atom reduce primitive on gfx950.
//
// "Purlin: Separating Orchestration from the Datapath of Collectives"
// (arXiv 2609.36954), abstract: the datapath provides a reduction primitive;
// Figure 4 (top) defines ReduceScatter as the sum of partition k over every
// input, and Figure 6 composes AllReduce from ReduceScatter and AllGather.
//
// One kernel family serves the flat reduce, ReduceScatter(V) and the fused
// one-shot AllReduce. Each lane owns 16-byte slots (8 bf16 or 4 fp32):
// it issues the P source loads of U slots back to back (P*U 128-bit loads
// in flight), widens to binary32, adds in rank order 0..P-1, rounds once to
// the element type and writes the slot to one output (ReduceScatter) or to
// every output (AllReduce: P stores of the same registers, so all outputs
// are bitwise identical by construction). Inputs are read once with
// non-temporal loads; outputs are streamed with non-temporal stores.
//
// Work is cut into tiles of blockDim.x * U slots within a part; a
// workgroup walks tiles with a grid stride. A part's last partial slot is
// reduced element by element by the lane that owns it.
#include "atom_dev.hpp"
#include "launch.hpp"

namespace atom {

namespace {

// Part of tile t: the last part whose first tile is <= t.
__device__ __forceinline__ int part_of_tile(const ReduceArgs& a, int64_t t)
{
    int k = 0;
    while (k + 1 < a.nparts && t >= a.tile_begin[k + 1])
        ++k;
    return k;
}

// Element-wise sum of element i (absolute index into every source).
template <typename T>
__device__ __forceinline__ float sum_elem(const ReduceArgs& a, int64_t i)
{
    float acc = Elem<T>::load(a.src[0], i);
    for (int r = 1; r < a.nsrc; ++r)
        acc = acc + Elem<T>::load(a.src[r], i);
    return acc;
}

template <typename T>
__device__ __forceinline__ void store_elem(const ReduceArgs& a, int k, int64_t pbeg, int64_t i,
                                           float v)
{
    if (a.mode == RM_SCATTER) {
        Elem<T>::store(a.dst[k], i - pbeg, v);
    } else {
        for (int q = 0; q < a.ndst; ++q)
            Elem<T>::store(a.dst[q], i, v);
    }
}

// GRID: the uniform form (grid_parts > 0). The part is blockIdx.y and the
// tile within it blockIdx.x, every part has part_off[1] elements starting at
// k * part_off[1], no head and the one shift shift[0]: nothing to look up
// before the loads. Otherwise tiles are numbered along a one-dimensional
// grid (grid-stride beyond its size) and each finds its part in tile_begin.
template <typename T, int P, int U, bool GRID>
__global__ __launch_bounds__(256) void k_reduce_vec(const ReduceArgs a)
{
    constexpr int VE = kVecBytes / sizeof(T);
    touch_arg_lines(&a.src[0], &a.src[8], &a.dst[0], &a.dst[8], &a.part_off[0], &a.tile_begin[0],
                    &a.ntiles, &a.head[0], &a.nsrc, hidden_args());
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const bool nt = a.nt_store != 0;
    const bool remap = a.xcd_remap != 0;
    const int64_t nloop = GRID ? 1 : a.ntiles;
    for (int64_t base = 0; base < nloop; base += gridDim.x) {
        int k;
        int64_t pstart, pend, tip;                             // tip: tile within the part
        int h;
        int32_t shift;
        if (GRID) {
            k = blockIdx.y;
            const int64_t L = a.part_off[1];
            pstart = static_cast<int64_t>(k) * L;
            pend = pstart + L;
            tip = blockIdx.x;
            h = 0;
            shift = a.shift[0];
        } else {
            const int64_t t = tile_of(base, remap);
            if (t >= a.ntiles)
                continue;
            k = part_of_tile(a, t);
            pstart = a.part_off[k];                            // the part's first element
            pend = a.part_off[k + 1];
            tip = t - a.tile_begin[k];
            h = a.head[k];
            shift = a.shift[k];
        }
        const int64_t pbeg = pstart + h;                       // its first 16-byte boundary
        const int64_t plen = pend - pbeg;                      // >= 0
        const int64_t nfull = plen / VE;                       // whole slots after the head
        // The head (elements before the boundary, when every stream of the
        // part is off alignment by the same amount) is reduced element by
        // element by the first lanes of the part's first tile.
        if (!GRID && tip == 0 && lane < h)
            store_elem<T>(a, k, pstart, pstart + lane, sum_elem<T>(a, pstart + lane));
        // First slot of the tile; the part's first tile may start before the
        // part (negative slots are skipped) so that tiles are aligned.
        const int64_t slot0 = tip * nthr * U - shift;
        // Uniform bases of this tile (one buffer resource per source, in
        // scalar registers, covering the tile); lanes add 32-bit offsets.
        const int64_t ebase = pbeg + slot0 * VE;                // absolute element index
        const uint32_t tile_bytes = static_cast<uint32_t>(nthr) * U * kVecBytes;
        __amdgpu_buffer_rsrc_t rs[P];
#pragma unroll
        for (int r = 0; r < P; ++r)
            rs[r] = stream_rsrc(static_cast<const char*>(a.src[r]) + ebase * sizeof(T), tile_bytes);

        u32x4 x[U][P];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t s = slot0 + u * nthr + lane;
            const uint32_t off = static_cast<uint32_t>(u * nthr + lane) * kVecBytes;
            if (s >= 0 && s < nfull) {
#pragma unroll
                for (int r = 0; r < P; ++r)
                    x[u][r] = ld16_stream(rs[r], off);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t s = slot0 + u * nthr + lane;
            const uint32_t off = static_cast<uint32_t>(u * nthr + lane) * kVecBytes;
            if (s >= 0 && s < nfull) {
                SlotAcc<T> acc;
                acc.init(x[u][0]);
#pragma unroll
                for (int r = 1; r < P; ++r)
                    acc.add(x[u][r]);
                const u32x4 y = acc.pack();
                if (a.mode == RM_SCATTER) {
                    char* db = static_cast<char*>(a.dst[k]) + (h + slot0 * VE) * sizeof(T);
                    st16(db, off, y, nt);
                } else {
                    for (int q = 0; q < a.ndst; ++q) {
                        char* db = static_cast<char*>(a.dst[q]) + ebase * sizeof(T);
                        st16(db, off, y, nt);
                    }
                }
            } else if (s == nfull && nfull * VE < plen) {
                // The part's last, partial slot.
                for (int64_t i = pbeg + nfull * VE; i < pbeg + plen; ++i)
                    store_elem<T>(a, k, pstart, i, sum_elem<T>(a, i));
            }
        }
    }
}

// Parts whose P sources sit at one offset from 16-byte alignment and whose
// destination(s) at another (ReduceScatterV with partitions of any length,
// outputs off alignment by a different amount): as k_copy_shift, tiles run
// over the part's aligned 16-byte source vectors (plus one), each lane
// reduces its vector of all P sources in rank order, takes the reduced
// vector below from its neighbour and writes the destination slot that
// straddles the two (element-wise at the part's two ends). Bytes of a vector
// outside the part are reduced too and never stored.
template <typename T, int P, int U>
__global__ __launch_bounds__(256) void k_reduce_shift(const ReduceArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const bool nt = a.nt_store != 0;
    for (int64_t base = 0; base < a.ntiles; base += gridDim.x) {
        const int64_t t = base + blockIdx.x;
        if (t >= a.ntiles)
            continue;
        const int k = part_of_tile(a, t);
        const int64_t tip = t - a.tile_begin[k];
        const int64_t pstart = a.part_off[k];
        const int64_t bytes = (a.part_off[k + 1] - pstart) * static_cast<int64_t>(sizeof(T));
        const char* s0 = static_cast<const char*>(a.src[0]) + pstart * sizeof(T);
        const int64_t A = static_cast<int64_t>(reinterpret_cast<uintptr_t>(s0));
        const int64_t vlo = A >> 4, vhi = (A + bytes - 1) >> 4;
        // Tiles are aligned to the tile size in the sources' address space,
        // so a wave's loads fill whole cache lines; the part's first tile may
        // start before it.
        const int64_t tv = static_cast<int64_t>(blockDim.x) * U;      // vectors per tile, a power of two
        const int64_t w0 = (vlo & ~(tv - 1)) + tip * tv + wave * 64 * U;
        const int64_t vofs = ((w0 - vlo) << 4) - (A & 15);     // source bytes of vector w0
        __amdgpu_buffer_rsrc_t rs[P];
#pragma unroll
        for (int r = 0; r < P; ++r)
            rs[r] = stream_rsrc(static_cast<const char*>(a.src[r]) + pstart * sizeof(T) + vofs,
                                64u * U * kVecBytes);
        u32x4 R[U], L[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = w0 + u * 64 + lane;
            R[u] = u32x4{0, 0, 0, 0};
            if (v >= vlo && v <= vhi) {
                const uint32_t off = static_cast<uint32_t>(u * 64 + lane) * kVecBytes;
                u32x4 x[P];
#pragma unroll
                for (int r = 0; r < P; ++r)
                    x[r] = ld16_stream(rs[r], off);
                SlotAcc<T> acc;
                acc.init(x[0]);
#pragma unroll
                for (int r = 1; r < P; ++r)
                    acc.add(x[r]);
                R[u] = acc.pack();
            }
        }
        u32x4 carry = {0, 0, 0, 0};
        if (lane == 0 && w0 - 1 >= vlo && w0 - 1 <= vhi) {
            SlotAcc<T> acc;
            acc.init(ld16_stream(static_cast<const char*>(a.src[0]) + pstart * sizeof(T) + vofs - kVecBytes));
            for (int r = 1; r < P; ++r)
                acc.add(ld16_stream(static_cast<const char*>(a.src[r]) + pstart * sizeof(T) + vofs - kVecBytes));
            carry = acc.pack();
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            L[u] = from_lane_below(R[u], u == 0 ? carry : lane63(R[u - 1]));
        const int q0 = a.mode == RM_SCATTER ? k : 0;
        const int q1 = a.mode == RM_SCATTER ? k + 1 : a.ndst;
        for (int q = q0; q < q1; ++q) {
            char* D = static_cast<char*>(a.dst[q]) + (a.mode == RM_SCATTER ? 0 : pstart * sizeof(T));
            const int d = static_cast<int>((reinterpret_cast<uintptr_t>(D) - static_cast<uint64_t>(A)) & 15);
            char* wbase = D + vofs - d;                          // 16-byte aligned
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t v = w0 + u * 64 + lane;
                const int64_t sa = (v << 4) - d;
                const int64_t lo = A - sa, hi = A + bytes - sa;
                const int p0 = lo > 0 ? static_cast<int>(lo) : 0;
                const int p1 = hi < 16 ? static_cast<int>(hi) : 16;
                if (v > vhi + 1 || p0 >= p1)
                    continue;
                const u32x4 slot = funnel16(L[u], R[u], d);
                const uint32_t off = static_cast<uint32_t>(u * 64 + lane) * kVecBytes;
                if (p0 == 0 && p1 == 16)
                    st16(wbase, off, slot, nt);
                else
                    store_slot_part(wbase + off, slot, p0, p1, static_cast<int>(sizeof(T)));
            }
        }
    }
}

// Element-wise variant for buffers or partitions off 16-byte alignment.
template <typename T>
__global__ __launch_bounds__(256) void k_reduce_elem(const ReduceArgs a)
{
    constexpr int VE = kVecBytes / sizeof(T);
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const bool remap = a.xcd_remap != 0;
    for (int64_t base = 0; base < a.ntiles; base += gridDim.x) {
        const int64_t t = tile_of(base, remap);
        if (t >= a.ntiles)
            continue;
        const int k = part_of_tile(a, t);
        const int64_t pbeg = a.part_off[k];
        const int64_t plen = a.part_off[k + 1] - pbeg;
        const int64_t slot0 = (t - a.tile_begin[k]) * nthr;    // U = 1 on this path
        const int64_t s = slot0 + lane;
        for (int e = 0; e < VE; ++e) {
            const int64_t i = s * VE + e;
            if (i < plen)
                store_elem<T>(a, k, pbeg, pbeg + i, sum_elem<T>(a, pbeg + i));
        }
    }
}

template <typename T, int P>
hipError_t launch_vec_p(const Plan& p, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(p.grid)), block(p.wg);
    if (p.ra.shifted) {
        if (p.ra.grid_parts != 0 || p.wg % 64 != 0)
            return hipErrorInvalidValue;
        switch (p.U) {
        case 1: k_reduce_shift<T, P, 1><<<grid, block, 0, stream>>>(p.ra); break;
        case 2:
            if constexpr (2 * P <= 32) { k_reduce_shift<T, P, 2><<<grid, block, 0, stream>>>(p.ra); break; }
            else return hipErrorInvalidValue;
        case 4:
            if constexpr (4 * P <= 32) { k_reduce_shift<T, P, 4><<<grid, block, 0, stream>>>(p.ra); break; }
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (p.ra.grid_parts > 0) {
        const dim3 g2(static_cast<unsigned>(p.grid), static_cast<unsigned>(p.ra.grid_parts));
        switch (p.U) {
        case 1: k_reduce_vec<T, P, 1, true><<<g2, block, 0, stream>>>(p.ra); break;
        case 2:
            if constexpr (2 * P <= 32) { k_reduce_vec<T, P, 2, true><<<g2, block, 0, stream>>>(p.ra); break; }
            else return hipErrorInvalidValue;
        case 4:
            if constexpr (4 * P <= 32) { k_reduce_vec<T, P, 4, true><<<g2, block, 0, stream>>>(p.ra); break; }
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (p.U) {
    case 1: k_reduce_vec<T, P, 1, false><<<grid, block, 0, stream>>>(p.ra); break;
    case 2:
        if constexpr (2 * P <= 32) { k_reduce_vec<T, P, 2, false><<<grid, block, 0, stream>>>(p.ra); break; }
        else return hipErrorInvalidValue;
    case 4:
        if constexpr (4 * P <= 32) { k_reduce_vec<T, P, 4, false><<<grid, block, 0, stream>>>(p.ra); break; }
        else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_vec(const Plan& p, hipStream_t stream)
{
    switch (p.P) {
    case 1: return launch_vec_p<T, 1>(p, stream);
    case 2: return launch_vec_p<T, 2>(p, stream);
    case 3: return launch_vec_p<T, 3>(p, stream);
    case 4: return launch_vec_p<T, 4>(p, stream);
    case 5: return launch_vec_p<T, 5>(p, stream);
    case 6: return launch_vec_p<T, 6>(p, stream);
    case 7: return launch_vec_p<T, 7>(p, stream);
    case 8: return launch_vec_p<T, 8>(p, stream);
    case 9: return launch_vec_p<T, 9>(p, stream);
    case 10: return launch_vec_p<T, 10>(p, stream);
    case 11: return launch_vec_p<T, 11>(p, stream);
    case 12: return launch_vec_p<T, 12>(p, stream);
    case 13: return launch_vec_p<T, 13>(p, stream);
    case 14: return launch_vec_p<T, 14>(p, stream);
    case 15: return launch_vec_p<T, 15>(p, stream);
    case 16: return launch_vec_p<T, 16>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_reduce(const Plan& p, hipStream_t stream)
{
    if (p.ra.nsrc != p.P || p.grid < 1 || p.wg < 1 || p.wg > 256)
        return hipErrorInvalidValue;
    if (p.ra.grid_parts != 0 &&
        (!p.vec || p.ra.grid_parts != p.ra.nparts || p.ra.grid_parts > 65535 || p.grid > 0x7fffffff))
        return hipErrorInvalidValue;
    if (p.vec) {
        // The vector path takes U from {1, 2, 4}; deeper requests are clamped
        // by the planner so that U * P 16-byte values fit in registers.
        return p.dtype == DT_BF16 ? launch_vec<uint16_t>(p, stream) : launch_vec<float>(p, stream);
    }
    const dim3 grid(static_cast<unsigned>(p.grid)), block(p.wg);
    if (p.dtype == DT_BF16)
        k_reduce_elem<uint16_t><<<grid, block, 0, stream>>>(p.ra);
    else
        k_reduce_elem<float><<<grid, block, 0, stream>>>(p.ra);
    return hipGetLastError();
}

}  // namespace atom
