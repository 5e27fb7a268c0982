// k_copy.hip -- the Atom copy primitive on gfx950.
//
// "Purlin: Separating Orchestration from the Datapath of Collectives"
// (arXiv 2609.36954), abstract: the datapath provides a copy primitive.
// Figure 4 gives the two copy layouts served here: AllGather (every rank
// receives every partition in rank order) and AllToAll (rank j receives
// partition j of every source, in source order); Table 2 adds their
// variable-length forms.
//
// The work is a list of segments, each a contiguous byte range of one
// source written to one destination (AllToAll(V)) or to every destination
// (AllGather(V), one load feeding P stores). Segment offsets are derived in
// the kernel from the row counts carried in the kernel arguments, so a
// launch needs no descriptor upload. Segments are cut into tiles of
// blockDim.x * U 16-byte slots; each lane issues its U loads back to back,
// then its stores (non-temporal: outputs are not re-read).
#include "atom_dev.hpp"
#include "launch.hpp"

namespace atom {

namespace {

struct Seg {
    const char* src;
    int64_t dst_off;   // byte offset in the destination(s)
    int64_t bytes;
    int dst;           // CK_EXCHANGE: destination index; CK_FANOUT: -1 (all)
};

// Largest s with seg_tile_begin[s] <= t (empty segments own no tile).
__device__ __forceinline__ int seg_of_tile(const CopyArgs& a, int64_t t)
{
    int lo = 0, hi = a.nseg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.seg_tile_begin[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ Seg seg_geometry(const CopyArgs& a, int s)
{
    Seg g;
    g.bytes = static_cast<int64_t>(a.cnt[s]) * a.row_bytes;
    if (a.kind == CK_FANOUT) {
        int64_t rows = 0;
        for (int k = 0; k < s; ++k)
            rows += a.cnt[k];
        g.src = static_cast<const char*>(a.src[s]);
        g.dst_off = rows * a.row_bytes;
        g.dst = -1;
    } else {
        const int r = s / a.P, j = s - r * a.P;
        int64_t src_rows = 0, dst_rows = 0;
        for (int jj = 0; jj < j; ++jj)       // source r's rows for earlier destinations
            src_rows += a.cnt[r * a.P + jj];
        for (int rr = 0; rr < r; ++rr)       // earlier sources' rows for destination j
            dst_rows += a.cnt[rr * a.P + j];
        g.src = static_cast<const char*>(a.src[r]) + src_rows * a.row_bytes;
        g.dst_off = dst_rows * a.row_bytes;
        g.dst = j;
    }
    return g;
}

template <typename W>
__device__ __forceinline__ void copy_units(const CopyArgs& a, const Seg& g, int64_t from, int64_t to)
{
    // Element-wise bytes [from, to) of the segment, in units of sizeof(W).
    for (int64_t b = from; b < to; b += sizeof(W)) {
        const W v = *reinterpret_cast<const W*>(g.src + b);
        if (g.dst >= 0) {
            *reinterpret_cast<W*>(static_cast<char*>(a.dst[g.dst]) + g.dst_off + b) = v;
        } else {
            for (int q = 0; q < a.ndst; ++q)
                *reinterpret_cast<W*>(static_cast<char*>(a.dst[q]) + g.dst_off + b) = v;
        }
    }
}

__device__ __forceinline__ void copy_bytes(const CopyArgs& a, const Seg& g, int64_t from, int64_t to)
{
    switch (a.esize) {
    case 4: copy_units<uint32_t>(a, g, from, to); break;
    case 2: copy_units<uint16_t>(a, g, from, to); break;
    default: copy_units<uint8_t>(a, g, from, to); break;
    }
}

// Geometry of segment s of the uniform form (every segment cnt[0] rows),
// computed without walking the counts.
__device__ __forceinline__ Seg seg_uniform(const CopyArgs& a, int s)
{
    Seg g;
    g.bytes = static_cast<int64_t>(a.cnt[0]) * a.row_bytes;
    if (a.kind == CK_FANOUT) {
        g.src = static_cast<const char*>(a.src[s]);
        g.dst_off = static_cast<int64_t>(s) * g.bytes;
        g.dst = -1;
    } else {
        const int r = s / a.P, j = s - r * a.P;
        g.src = static_cast<const char*>(a.src[r]) + static_cast<int64_t>(j) * g.bytes;
        g.dst_off = static_cast<int64_t>(r) * g.bytes;
        g.dst = j;
    }
    return g;
}

// HEADS: some segment starts off a 16-byte boundary (instantiated apart so
// that aligned plans run without the per-tile head check). GRID: the uniform
// form (grid_segs > 0): the segment is blockIdx.y and the tile within it
// blockIdx.x, so nothing is looked up before the loads.
template <int U, bool HEADS, bool GRID>
__global__ __launch_bounds__(256) void k_copy_vec(const CopyArgs a)
{
    static_assert(!(HEADS && GRID), "the uniform form has no heads");
    touch_arg_lines(&a.src[0], &a.src[8], &a.dst[0], &a.dst[8], &a.row_bytes, &a.seg_off[0],
                    &a.cnt[0], &a.seg_tile_begin[0], &a.head[0], hidden_args());
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const bool nt = a.nt_store != 0;
    const bool remap = a.xcd_remap != 0;
    const int64_t nloop = GRID ? 1 : a.ntiles;
    for (int64_t base = 0; base < nloop; base += gridDim.x) {
        int s;
        int64_t tip;                                      // tile within the segment
        if (GRID) {
            s = blockIdx.y;
            tip = blockIdx.x;
        } else {
            const int64_t t = tile_of(base, remap);
            if (t >= a.ntiles)
                continue;
            s = seg_of_tile(a, t);
            tip = t - a.seg_tile_begin[s];
        }
        Seg g = GRID ? seg_uniform(a, s) : seg_geometry(a, s);
        // The segment's head (bytes before the first 16-byte boundary, when
        // its source and destinations are off alignment by the same amount)
        // is copied element by element by the first lanes of its first tile;
        // the tiles then cover the rest from that boundary.
        const int h = HEADS ? a.head[s] : 0;
        if (HEADS && h > 0) {
            if (tip == 0 && lane * a.esize < h)
                copy_bytes(a, g, static_cast<int64_t>(lane) * a.esize,
                           static_cast<int64_t>(lane + 1) * a.esize);
            g.src += h;
            g.dst_off += h;
            g.bytes -= h;
        }
        // Tile start in the segment; the first tile may start before the
        // segment (negative offsets are skipped) so that tiles are aligned
        // at the destination.
        int64_t b0 = tip * a.tile_bytes;
        if (a.align) {
            const char* d = static_cast<const char*>(a.dst[g.dst >= 0 ? g.dst : 0]) + g.dst_off;
            b0 -= seg_tile_shift(reinterpret_cast<uintptr_t>(d), a.tile_bytes);
        }
        const char* sb = g.src + b0;
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t o = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
            if (o >= 0 && o + kVecBytes <= g.bytes)
                x[u] = ld16_stream(sb + static_cast<uint32_t>(u * nthr + lane) * kVecBytes);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t off = static_cast<uint32_t>(u * nthr + lane) * kVecBytes;
            const int64_t o = b0 + off;
            if (o < 0) {
                // before the segment: owned by no lane
            } else if (o + kVecBytes <= g.bytes) {
                if (g.dst >= 0) {
                    char* db = static_cast<char*>(a.dst[g.dst]) + g.dst_off + b0;
                    st16(db, off, x[u], nt);
                } else {
                    for (int q = 0; q < a.ndst; ++q) {
                        char* db = static_cast<char*>(a.dst[q]) + g.dst_off + b0;
                        st16(db, off, x[u], nt);
                    }
                }
            } else if (o < g.bytes) {
                copy_bytes(a, g, o, g.bytes);   // the segment's last, partial slot
            }
        }
    }
}

// Fan-out in blocked order (AllGather(V) beyond the latency path). One load
// feeding P stores keeps P write streams open at once across the chip, and
// measured on MI355X that pattern writes at 5.2-5.7 TB/s where one stream
// writes at 6.6. Here the tiles are cut into blocks of 2^block_shift
// consecutive tiles; workgroup task w takes (block, output, tile) with the
// output varying slower than the tile within a block, so at any time the
// chip writes one output's part of one block. The block size and the grid
// are multiples of the 8 XCDs, and workgroup w runs on XCD w mod 8, so tile i
// of a block runs on XCD i mod 8 for every output: its source bytes, read
// from memory by the first output's pass, are read again from that XCD's L2
// by the others (the block is sized so that its share per XCD stays in the
// L2, and the loads are ordinary ones: a streaming load would not keep the
// line, measured 7.5x the source bytes read from memory instead of 1x).
// Each workgroup loads its tile once and stores it to one output. Every wave
// runs the task decode on the scalar unit, which one SIMD shares among its
// waves, so the decode is kept to shifts, one 32-bit division and a short
// search (64-bit divisions there took the kernel from 6.0 to 3.4 TB/s).
template <int U, bool HEADS>
__global__ __launch_bounds__(256) void k_copy_fan_blocked(const CopyArgs a)
{
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const bool nt = a.nt_store != 0;
    const uint32_t lb = static_cast<uint32_t>(a.block_shift);
    const uint32_t nd = static_cast<uint32_t>(a.ndst);
    for (int64_t w = blockIdx.x; w < a.nwork; w += gridDim.x) {
        const uint32_t u = static_cast<uint32_t>(static_cast<uint64_t>(w) >> lb);  // block * ndst + output
        const uint32_t blk = u / nd;
        const int q = static_cast<int>(u - blk * nd);
        const int64_t t = (static_cast<int64_t>(blk) << lb) + (w & ((int64_t(1) << lb) - 1));
        if (t >= a.ntiles)
            continue;
        int s = 0;                                   // segment: last with seg_tile_begin <= t
        while (s + 1 < a.nseg && a.seg_tile_begin[s + 1] <= t)
            ++s;
        const int64_t tip = t - a.seg_tile_begin[s];
        Seg g;
        g.src = static_cast<const char*>(a.src[s]);
        g.dst_off = a.seg_off[s];
        g.bytes = a.seg_off[s + 1] - a.seg_off[s];
        g.dst = q;                                   // this workgroup's one output
        const int h = HEADS ? a.head[s] : 0;
        if (HEADS && h > 0) {
            if (tip == 0 && lane * a.esize < h)
                copy_bytes(a, g, static_cast<int64_t>(lane) * a.esize,
                           static_cast<int64_t>(lane + 1) * a.esize);
            g.src += h;
            g.dst_off += h;
            g.bytes -= h;
        }
        // Tiles are aligned to the tile size at output 0, as the planner
        // counted them; the tiles are the same byte ranges for every output.
        int64_t b0 = tip * a.tile_bytes;
        if (a.align)
            b0 -= seg_tile_shift(reinterpret_cast<uintptr_t>(static_cast<const char*>(a.dst[0]) + g.dst_off),
                                 a.tile_bytes);
        const char* sb = g.src + b0;
        u32x4 x[U];
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const int64_t o = b0 + static_cast<int64_t>(uu * nthr + lane) * kVecBytes;
            if (o >= 0 && o + kVecBytes <= g.bytes)
                x[uu] = ld16(sb + static_cast<uint32_t>(uu * nthr + lane) * kVecBytes);
        }
        char* db = static_cast<char*>(a.dst[q]) + g.dst_off + b0;
#pragma unroll
        for (int uu = 0; uu < U; ++uu) {
            const uint32_t off = static_cast<uint32_t>(uu * nthr + lane) * kVecBytes;
            const int64_t o = b0 + off;
            if (o < 0) {
                // before the segment: owned by no lane
            } else if (o + kVecBytes <= g.bytes) {
                st16(db, off, x[uu], nt);
            } else if (o < g.bytes) {
                copy_bytes(a, g, o, g.bytes);      // the segment's last, partial slot
            }
        }
    }
}

// Segments whose source and destinations sit at different offsets from
// 16-byte alignment (a V collective with rows of any length, buffers off
// alignment by different amounts). Tiles run over the segment's 16-byte
// source vectors, aligned in the address space: vector v holds bytes
// [16v, 16v + 16), from the one holding the segment's first byte to one past
// the one holding its last. Each wave owns 64 * U consecutive vectors, lane
// l of row u vector v = w0 + 64u + l; it loads v (ordinary 16-byte loads,
// which stay inside blocks that hold segment bytes), takes v - 1 from the
// lane below (lane 0 from the previous row, or a load of its own for the
// wave's first vector), and writes the destination slot that holds the
// tail of v - 1 and the head of v: a 16-byte aligned store, or element-wise
// stores for the slots at the segment's two ends. Every destination of a
// segment sits at the same offset d from the source modulo 16.
template <int U>
__global__ __launch_bounds__(256) void k_copy_shift(const CopyArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const bool nt = a.nt_store != 0;
    for (int64_t base = 0; base < a.ntiles; base += gridDim.x) {
        const int64_t t = base + blockIdx.x;
        if (t >= a.ntiles)
            continue;
        const int s = seg_of_tile(a, t);
        const int64_t tip = t - a.seg_tile_begin[s];
        const Seg g = seg_geometry(a, s);
        const int64_t A = static_cast<int64_t>(reinterpret_cast<uintptr_t>(g.src));
        const int64_t vlo = A >> 4, vhi = (A + g.bytes - 1) >> 4;
        // Tiles are aligned to the tile size in the address space, at the
        // source (exchange) or at output 0 (fan-out: P stores per load), so
        // a wave's 16-byte accesses on that side fill whole cache lines; the
        // first tile may start before the segment.
        const int64_t tv = static_cast<int64_t>(blockDim.x) * U;      // vectors per tile, a power of two
        int64_t v0 = vlo & ~(tv - 1);
        if (a.align) {
            const int64_t m0 = static_cast<int64_t>(reinterpret_cast<uintptr_t>(static_cast<const char*>(a.dst[0]) + g.dst_off)) - A;
            v0 = vlo - ((vlo + (m0 >> 4)) & (tv - 1));
        }
        const int64_t w0 = v0 + tip * tv + wave * 64 * U;
        // vector v at g.src - (A & 15) + 16 (v - vlo): addresses derived from
        // the argument pointer, so the loads are global (not flat) ones
        const char* vb = g.src - (A & 15) + ((w0 - vlo) << 4);
        u32x4 R[U], L[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = w0 + u * 64 + lane;
            R[u] = v >= vlo && v <= vhi ? ld16(vb + (u * 64 + lane) * kVecBytes) : u32x4{0, 0, 0, 0};
        }
        u32x4 carry = {0, 0, 0, 0};
        if (lane == 0 && w0 - 1 >= vlo && w0 - 1 <= vhi)
            carry = ld16(vb - kVecBytes);
#pragma unroll
        for (int u = 0; u < U; ++u)
            L[u] = from_lane_below(R[u], u == 0 ? carry : lane63(R[u - 1]));
        const int q0 = g.dst >= 0 ? g.dst : 0;
        const int q1 = g.dst >= 0 ? g.dst + 1 : a.ndst;
        for (int q = q0; q < q1; ++q) {
            char* D = static_cast<char*>(a.dst[q]) + g.dst_off;
            const int d = static_cast<int>((reinterpret_cast<uintptr_t>(D) - static_cast<uint64_t>(A)) & 15);
            // slot of vector v: source bytes [16v - d, 16v - d + 16), written
            // 16-byte aligned at D + 16 (v - vlo) - (A & 15) - d; wave-uniform base
            char* wbase = D + ((w0 - vlo) << 4) - (A & 15) - d;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t v = w0 + u * 64 + lane;
                const int64_t sa = (v << 4) - d;
                const int64_t lo = A - sa, hi = A + g.bytes - sa;
                const int p0 = lo > 0 ? static_cast<int>(lo) : 0;
                const int p1 = hi < 16 ? static_cast<int>(hi) : 16;
                if (v > vhi + 1 || p0 >= p1)
                    continue;
                const u32x4 slot = funnel16(L[u], R[u], d);
                const uint32_t off = static_cast<uint32_t>(u * 64 + lane) * kVecBytes;
                if (p0 == 0 && p1 == 16)
                    st16(wbase, off, slot, nt);
                else
                    store_slot_part(wbase + off, slot, p0, p1, a.esize);
            }
        }
    }
}

// Element-wise variant for unaligned buffers or rows (U = 1).
__global__ __launch_bounds__(256) void k_copy_elem(const CopyArgs a)
{
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const bool remap = a.xcd_remap != 0;
    for (int64_t base = 0; base < a.ntiles; base += gridDim.x) {
        const int64_t t = tile_of(base, remap);
        if (t >= a.ntiles)
            continue;
        const int s = seg_of_tile(a, t);
        const Seg g = seg_geometry(a, s);
        const int64_t o = (t - a.seg_tile_begin[s]) * a.tile_bytes + static_cast<int64_t>(lane) * kVecBytes;
        if (o < g.bytes)
            copy_bytes(a, g, o, o + kVecBytes < g.bytes ? o + kVecBytes : g.bytes);
    }
    (void)nthr;
}

}  // namespace

hipError_t launch_copy(const Plan& p, hipStream_t stream)
{
    if (p.grid < 1 || p.wg < 1 || p.wg > 256 || p.ca.nseg < 1)
        return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(p.grid)), block(p.wg);
    if (!p.vec) {
        if (p.U != 1)
            return hipErrorInvalidValue;
        k_copy_elem<<<grid, block, 0, stream>>>(p.ca);
        return hipGetLastError();
    }
    if (p.ca.shifted) {
        if (p.ca.block_shift >= 0 || p.ca.grid_segs != 0 || p.wg % 64 != 0)
            return hipErrorInvalidValue;
        switch (p.U) {
        case 1: k_copy_shift<1><<<grid, block, 0, stream>>>(p.ca); break;
        case 2: k_copy_shift<2><<<grid, block, 0, stream>>>(p.ca); break;
        case 4: k_copy_shift<4><<<grid, block, 0, stream>>>(p.ca); break;
        case 8: k_copy_shift<8><<<grid, block, 0, stream>>>(p.ca); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    bool heads = false;
    for (int s = 0; s < p.ca.nseg; ++s)
        heads = heads || p.ca.head[s] != 0;
    if (p.ca.block_shift >= 0) {
        if (p.ca.kind != CK_FANOUT || p.ca.grid_segs != 0 || p.ca.nseg > kMaxRanks ||
            p.ca.block_shift > 30 || p.ca.ndst < 1 ||
            (p.ca.nwork >> p.ca.block_shift) > 0xFFFFFFFFll)
            return hipErrorInvalidValue;
#define ATOM_COPY_BLK(UU)                                                    \
    case UU:                                                                 \
        if (heads)                                                           \
            k_copy_fan_blocked<UU, true><<<grid, block, 0, stream>>>(p.ca);  \
        else                                                                 \
            k_copy_fan_blocked<UU, false><<<grid, block, 0, stream>>>(p.ca); \
        break;
        switch (p.U) {
        ATOM_COPY_BLK(1) ATOM_COPY_BLK(2) ATOM_COPY_BLK(4) ATOM_COPY_BLK(8)
        default: return hipErrorInvalidValue;
        }
#undef ATOM_COPY_BLK
        return hipGetLastError();
    }
    const int gs = p.ca.grid_segs;
    if (gs != 0 && (gs != p.ca.nseg || gs > 65535 || heads || p.grid > 0x7fffffff))
        return hipErrorInvalidValue;
    const dim3 grid2(static_cast<unsigned>(p.grid), static_cast<unsigned>(gs > 0 ? gs : 1));
#define ATOM_COPY_VEC(UU)                                                  \
    case UU:                                                               \
        if (gs > 0)                                                        \
            k_copy_vec<UU, false, true><<<grid2, block, 0, stream>>>(p.ca); \
        else if (heads)                                                    \
            k_copy_vec<UU, true, false><<<grid, block, 0, stream>>>(p.ca); \
        else                                                               \
            k_copy_vec<UU, false, false><<<grid, block, 0, stream>>>(p.ca); \
        break;
    switch (p.U) {
    ATOM_COPY_VEC(1) ATOM_COPY_VEC(2) ATOM_COPY_VEC(4) ATOM_COPY_VEC(8)
    default: return hipErrorInvalidValue;
    }
#undef ATOM_COPY_VEC
    return hipGetLastError();
}

}  // namespace atom
