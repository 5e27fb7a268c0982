// plan.cpp -- host planner of libatom.
//
// From "Purlin: Separating Orchestration from the Datapath of Collectives"
// (arXiv 2609.36954): the abstract defines a collective by its input
// layout, its output layout and a copy or reduce operation, and the
// derivability row of Table 1 wants the orchestration to follow from that
// definition, with no hand-written schedule. This file is that derivation:
// the layout pair and op select the collective (Figure 4, Figure 6,
// Table 2), the buffer shapes follow from the partition size or the counts,
// and the launch (tiles, grid, SNAC chunks) follows from the shapes.
#include "plan.hpp"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>

namespace atom {

namespace {

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

int esize_of(atom_dtype d)
{
    switch (d) {
    case ATOM_DT_BF16: return 2;
    case ATOM_DT_F32: return 4;
    default: return 0;
    }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// a*b without overflow, for non-negative operands; false on overflow.
bool mul_ok(int64_t a, int64_t b, int64_t* out)
{
    if (a < 0 || b < 0)
        return false;
    if (a != 0 && b > INT64_MAX / a)
        return false;
    *out = a * b;
    return true;
}

struct Cfg {
    int64_t chunk;
    bool chunk_set;    // chunk given by the caller
    int32_t stages;    // 0 = pick by shape
    int64_t num_wgs;   // 0 = pick by shape
    uint32_t flags;
    int32_t slots;
    bool slots_set;    // ring depth given by the caller
    int64_t piece;     // SNAC task granule; 0 = default
    int64_t wait_us;   // bound of one SNAC wait
    int32_t lanes;     // threads per workgroup; 0 = pick by shape
    int64_t jitter_us; // SNAC test hook: largest delay before a notify or consume
    uint32_t jitter_seed;
    int32_t lead;      // SNAC: chunks staged ahead of the consumers; 0 = ring depth
    unsigned long long* trace;  // SNAC measurement hook (NULL: off)
};

atom_status read_cfg(const atom_config* cfg, Cfg* c)
{
    c->chunk = 0;          // staged chunk: chosen per collective unless given
    c->chunk_set = false;
    c->stages = 0;
    c->num_wgs = 0;
    c->flags = 0;
    c->slots = kDefaultSlots;
    c->slots_set = false;
    c->piece = 0;
    c->wait_us = kDefaultWaitUs;
    c->lanes = 0;
    c->jitter_us = 0;
    c->jitter_seed = 0;
    c->lead = 0;
    c->trace = nullptr;
    if (!cfg)
        return ATOM_OK;
    if (cfg->chunk_bytes != 0) {
        if (!is_pow2(cfg->chunk_bytes) || cfg->chunk_bytes < kMinChunk || cfg->chunk_bytes > kMaxChunk)
            return ATOM_ERR_INVALID_ARG;
        c->chunk = cfg->chunk_bytes;
        c->chunk_set = true;
    }
    if (cfg->stages != 0) {
        if (cfg->stages != 1 && cfg->stages != 2 && cfg->stages != 4 && cfg->stages != 8)
            return ATOM_ERR_INVALID_ARG;
        c->stages = cfg->stages;
    }
    if (cfg->num_wgs < 0)
        return ATOM_ERR_INVALID_ARG;
    c->num_wgs = std::min<int64_t>(cfg->num_wgs, kMaxGrid);
    if (cfg->flags & ~(ATOM_F_STAGED | ATOM_F_NO_NT | ATOM_F_XCD_ORDER | ATOM_F_COUNTED))
        return ATOM_ERR_INVALID_ARG;
    c->flags = cfg->flags;
    if (cfg->ring_slots != 0) {
        if (cfg->ring_slots < 1 || cfg->ring_slots > kMaxSlots)
            return ATOM_ERR_INVALID_ARG;
        c->slots = cfg->ring_slots;
        c->slots_set = true;
    }
    if (cfg->piece_bytes != 0) {
        if (!is_pow2(cfg->piece_bytes) || cfg->piece_bytes < (16 << 10) || cfg->piece_bytes > kMaxChunk)
            return ATOM_ERR_INVALID_ARG;
        c->piece = cfg->piece_bytes;
    }
    if (cfg->wait_us < 0)
        return ATOM_ERR_INVALID_ARG;
    if (cfg->wait_us > 0)
        c->wait_us = cfg->wait_us;
    if (cfg->lanes != 0 && cfg->lanes != 64 && cfg->lanes != 128 && cfg->lanes != 256 &&
        cfg->lanes != 512)
        return ATOM_ERR_INVALID_ARG;
    // 512 lanes exist only for the staged (SNAC) kernel
    if (cfg->lanes > 256 && !(cfg->flags & ATOM_F_STAGED))
        return ATOM_ERR_UNSUPPORTED;
    c->lanes = cfg->lanes;
    if (cfg->jitter_us < 0 || cfg->jitter_us > kMaxJitterUs)
        return ATOM_ERR_INVALID_ARG;
    c->jitter_us = cfg->jitter_us;
    c->jitter_seed = cfg->jitter_seed;
    if (cfg->snac_lead < 0 || cfg->snac_lead > kMaxSlots)
        return ATOM_ERR_INVALID_ARG;
    c->lead = cfg->snac_lead;
    c->trace = reinterpret_cast<unsigned long long*>(cfg->trace);
    return ATOM_OK;
}

// Outputs must be pairwise disjoint and disjoint from every input; inputs
// may alias each other (they are only read). Empty ranges never overlap.
bool disjoint(const Range* ins, int nin, const Range* outs, int nout)
{
    for (int o = 0; o < nout; ++o) {
        if (outs[o].lo == outs[o].hi)
            continue;
        for (int i = 0; i < nin; ++i)
            if (ins[i].lo != ins[i].hi && outs[o].lo < ins[i].hi && ins[i].lo < outs[o].hi)
                return false;
        for (int q = o + 1; q < nout; ++q)
            if (outs[q].lo != outs[q].hi && outs[o].lo < outs[q].hi && outs[q].lo < outs[o].hi)
                return false;
    }
    return true;
}

Range range_of(const void* p, int64_t bytes)
{
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

// A buffer is usable when it is element-aligned, and non-NULL unless empty.
bool buffer_ok(const void* p, int64_t bytes, int esize)
{
    if (bytes == 0)
        return true;
    return p != nullptr && aligned(p, static_cast<uintptr_t>(esize));
}

// 16-byte slots per lane per tile (the Atom pipeline depth), for the
// 64-lane workgroups of the vector path. Measured on MI355X with one tile
// per workgroup: many small tiles keep the most bytes in flight, so one
// slot per lane wins for the scatter-reduce, the fused AllReduce and the
// fan-out copy, two for the exchange (AllToAll(V)) and for reduces of at
// most 4 sources; the flat copy uses 128-lane tiles of two slots per lane.
// The reduce kernel is built for U in {1, 2, 4} with U * P <= 32.
int32_t pick_u_reduce(int nsrc, int32_t mode, int32_t stages)
{
    int32_t u = stages ? std::min<int32_t>(stages, 4)
                       : (mode == RM_FANOUT ? 1 : (nsrc <= 4 ? 2 : 1));
    while (u > 1 && u * nsrc > 32)
        u /= 2;
    return u;
}

int32_t pick_u_copy(int32_t kind, int nseg, int32_t stages)
{
    if (stages)
        return stages;
    if (nseg == 1)
        return 2;                           // one flat copy: 4 KiB tiles
    return kind == CK_FANOUT ? 1 : 2;       // AllGather fan-out / AllToAll(V) exchange
}

int64_t pick_grid(int64_t ntiles, int64_t num_wgs)
{
    int64_t g = num_wgs > 0 ? num_wgs : kMaxGrid;
    return std::max<int64_t>(1, std::min(ntiles, g));
}

// Reduce family launch from part boundaries (elements).
void build_reduce(Plan* p, int nsrc, const void* const* srcs, int ndst, void* const* dsts,
                  int nparts, const int64_t* part_off, int32_t mode, const Cfg& c)
{
    ReduceArgs& a = p->ra;
    std::memset(&a, 0, sizeof a);
    const int es = p->esize;
    for (int r = 0; r < nsrc; ++r)
        a.src[r] = srcs[r];
    for (int q = 0; q < ndst; ++q)
        a.dst[q] = dsts[q];
    for (int k = 0; k <= nparts; ++k)
        a.part_off[k] = part_off[k];
    // Vector path: within each part every stream (its P sources and its
    // destinations) sits at the same offset from 16-byte alignment. Then the
    // elements before the first boundary (the head) are reduced one by one
    // and the rest in 16-byte slots; otherwise the element-wise kernel runs.
    auto mis = [](const void* b, int64_t byte_off) {
        return static_cast<unsigned>((reinterpret_cast<uintptr_t>(b) + static_cast<uint64_t>(byte_off)) %
                                     kVecBytes);
    };
    bool vec = true;
    for (int k = 0; k < nparts && vec; ++k) {
        const int64_t off = part_off[k] * es;
        const unsigned d = mis(srcs[0], off);
        for (int r = 1; r < nsrc; ++r)
            vec = vec && mis(srcs[r], off) == d;
        if (mode == RM_SCATTER)
            vec = vec && mis(dsts[k], 0) == d;
        else
            for (int q = 0; q < ndst; ++q)
                vec = vec && mis(dsts[q], off) == d;
        const int64_t len = part_off[k + 1] - part_off[k];
        a.head[k] = static_cast<int32_t>(std::min<int64_t>(len, ((kVecBytes - d) % kVecBytes) / es));
    }
    if (!vec)
        std::memset(a.head, 0, sizeof a.head);
    // Shifted vector path (k_reduce_shift): each part's sources share one
    // offset from 16-byte alignment and its destination(s) share another.
    // Only when that fails for a part does the call run element by element.
    bool shifted = false;
    if (!vec) {
        shifted = true;
        for (int k = 0; k < nparts && shifted; ++k) {
            const int64_t off = part_off[k] * es;
            const unsigned d = mis(srcs[0], off);
            for (int r = 1; r < nsrc; ++r)
                shifted = shifted && mis(srcs[r], off) == d;
            if (mode == RM_FANOUT)
                for (int q = 1; q < ndst; ++q)
                    shifted = shifted && mis(dsts[q], off) == mis(dsts[0], off);
        }
        vec = shifted;
    }
    a.shifted = shifted ? 1 : 0;
    const int64_t ve = kVecBytes / es;   // elements per 16-byte slot
    p->vec = vec ? 1 : 0;
    p->U = vec ? pick_u_reduce(nsrc, mode, c.stages) : 1;
    // The vector path streams best from many small tiles: 64-lane
    // workgroups measured +8% over 256 lanes on a cold 8-way reduce and +5%
    // on the fused AllReduce on MI355X.
    p->wg = vec ? 64 : 256;
    // The shifted path: 64 lanes x 2 slots measured best on MI355X (the
    // Zipf ReduceScatterV of 8 x 256 MiB in single-element partitions:
    // 5.68 TB/s, against 5.40 with one slot and 5.25-5.66 at 128-256 lanes).
    if (shifted && !c.stages && 2 * nsrc <= 32)
        p->U = 2;
    int64_t slots = 0;
    for (int k = 0; k < nparts; ++k)
        slots += ceil_div(part_off[k + 1] - part_off[k], ve);
    if (slots < kSmallSlots && !c.stages) {
        // Latency path: spread a small message over as many CUs as it can
        // use (one slot per lane, 64-lane workgroups).
        p->U = 1;
        p->wg = 64;
    }
    if (c.lanes)
        p->wg = c.lanes;
    const int64_t slots_per_tile = static_cast<int64_t>(p->wg) * p->U;
    int64_t t = 0;
    for (int k = 0; k < nparts; ++k) {
        a.tile_begin[k] = t;
        const int64_t len = part_off[k + 1] - part_off[k] - a.head[k];
        // Vector path: start tiles at addresses aligned to the tile size in
        // source 0 (a part that starts mid-tile gets a short first tile), so
        // a tile's loads never straddle two tile-sized blocks of memory.
        int64_t shift = 0;
        if (vec && !shifted) {
            const uint64_t addr = reinterpret_cast<uintptr_t>(srcs[0]) +
                                  static_cast<uint64_t>((part_off[k] + a.head[k]) * es);
            shift = seg_tile_shift(addr, slots_per_tile * kVecBytes) / kVecBytes;
        }
        a.shift[k] = static_cast<int32_t>(shift);
        int64_t tiles = ceil_div(ceil_div(len, ve) + shift, slots_per_tile);
        if (a.head[k] > 0 && tiles == 0)
            tiles = 1;                   // a part that is all head still needs its tile
        if (shifted && len > 0) {
            // the part's source vectors, plus one for the last slot, from the
            // tile-aligned vector at or before its first
            const uint64_t a0 = reinterpret_cast<uintptr_t>(srcs[0]) + static_cast<uint64_t>(part_off[k] * es);
            const int64_t vlo = static_cast<int64_t>(a0 / kVecBytes);
            const int64_t nv = static_cast<int64_t>((a0 + len * es - 1) / kVecBytes) + 2 -
                               (vlo & ~(slots_per_tile - 1));
            tiles = ceil_div(nv, slots_per_tile);
        }
        t += tiles;
    }
    a.tile_begin[nparts] = t;
    a.ntiles = t;
    a.nsrc = nsrc;
    a.ndst = ndst;
    a.nparts = nparts;
    a.mode = mode;
    // Streaming stores for outputs that are not re-read soon; a message on
    // the latency path is small and typically read by the next operation, so
    // its outputs stay in the caches for that reader (the call itself takes
    // the same time either way on MI355X: 3.3 us back to back for the decode
    // AllReduce).
    a.nt_store = ((c.flags & ATOM_F_NO_NT) || slots < kSmallSlots) ? 0 : 1;
    a.xcd_remap = (c.flags & ATOM_F_XCD_ORDER) ? 1 : 0;
    p->grid = pick_grid(t, c.num_wgs);
    p->exec = t > 0 ? EX_REDUCE : EX_NONE;
    // Uniform form of the latency path: equal parts laid end to end, no
    // heads, one shift, one tile per workgroup. The grid is then
    // tiles-per-part x parts and a workgroup knows its part and tile from
    // its coordinates, with no walk through the part table before its first
    // load. Measured on MI355X: the decode AllReduce (8 x b x 7168 bf16)
    // went from 3.36 to 3.10 us per call back to back. For large messages
    // the two grids measured within noise of each other (8-way
    // ReduceScatter of 8 x 256 MiB: 6.25-6.37 against 6.29-6.33 TB/s), so
    // they keep the one-dimensional grid and its grid-stride loop.
    a.grid_parts = 0;
    const int64_t L = part_off[1] - part_off[0];
    const int64_t tpp = nparts > 0 ? a.tile_begin[1] : 0;
    bool uniform = vec && !shifted && t > 0 && slots < kSmallSlots && part_off[0] == 0 && !a.xcd_remap &&
                   c.num_wgs == 0 && t <= kMaxGrid && nparts <= 65535;
    for (int k = 0; k < nparts && uniform; ++k)
        uniform = part_off[k] == k * L && a.head[k] == 0 && a.shift[k] == a.shift[0] &&
                  a.tile_begin[k] == k * tpp;
    if (uniform) {
        a.grid_parts = nparts;
        p->grid = tpp;
    }
}

// Copy family launch. cnt[s] rows of row_bytes per segment.
void build_copy(Plan* p, int32_t kind, int P, const void* const* srcs, int nsrc,
                void* const* dsts, int ndst, const int64_t* cnt, int nseg, int64_t row_bytes,
                int esize, const Cfg& c)
{
    CopyArgs& a = p->ca;
    std::memset(&a, 0, sizeof a);
    for (int r = 0; r < nsrc; ++r)
        a.src[r] = srcs[r];
    for (int q = 0; q < ndst; ++q)
        a.dst[q] = dsts[q];
    // Segment geometry (as the kernel derives it): source address and
    // destination byte offset of every segment.
    uint64_t seg_src[kMaxSegs], seg_dst[kMaxSegs];    // dst: of dsts[0] (fan-out) or dsts[j]
    if (kind == CK_FANOUT) {
        int64_t rows_before = 0;
        for (int s = 0; s < nseg; ++s) {
            seg_src[s] = reinterpret_cast<uintptr_t>(srcs[s]);
            seg_dst[s] = static_cast<uint64_t>(rows_before * row_bytes);
            rows_before += cnt[s];
        }
    } else {
        int64_t col_rows[kMaxRanks] = {};              // rows already bound for j
        for (int r = 0; r < P; ++r) {
            int64_t src_rows = 0;                      // rows of source r before j
            for (int j = 0; j < P; ++j) {
                const int s = r * P + j;
                seg_src[s] = reinterpret_cast<uintptr_t>(srcs[r]) + static_cast<uint64_t>(src_rows * row_bytes);
                seg_dst[s] = static_cast<uint64_t>(col_rows[j] * row_bytes);
                src_rows += cnt[s];
                col_rows[j] += cnt[s];
            }
        }
    }
    // Vector path: within each segment the source and every destination sit
    // at the same offset from 16-byte alignment; the bytes before the first
    // boundary (the head) are copied element by element, the rest in 16-byte
    // slots. Otherwise the element-wise kernel runs.
    bool aligned_all = row_bytes % kVecBytes == 0 || nseg == 1;
    for (int r = 0; r < nsrc; ++r)
        aligned_all = aligned_all && aligned(srcs[r], kVecBytes);
    for (int q = 0; q < ndst; ++q)
        aligned_all = aligned_all && aligned(dsts[q], kVecBytes);
    bool vec = true;
    for (int s = 0; s < nseg && vec && !aligned_all; ++s) {
        const int64_t bytes_s = cnt[s] * row_bytes;
        if (bytes_s == 0)
            continue;
        const unsigned d = static_cast<unsigned>(seg_src[s] % kVecBytes);
        if (kind == CK_FANOUT) {
            for (int q = 0; q < ndst; ++q)
                vec = vec && (reinterpret_cast<uintptr_t>(dsts[q]) + seg_dst[s]) % kVecBytes == d;
        } else {
            vec = vec && (reinterpret_cast<uintptr_t>(dsts[s % P]) + seg_dst[s]) % kVecBytes == d;
        }
        a.head[s] = static_cast<uint8_t>(std::min<int64_t>(bytes_s, (kVecBytes - d) % kVecBytes));
    }
    if (!vec)
        std::memset(a.head, 0, sizeof a.head);
    // Shifted vector path (k_copy_shift): a segment's source and its
    // destinations sit at different offsets from 16-byte alignment, every
    // destination of the segment at the same one. Only when that fails for a
    // segment does the whole call run element by element.
    bool shifted = false;
    if (!vec) {
        shifted = true;
        for (int s = 0; s < nseg && shifted; ++s) {
            if (cnt[s] * row_bytes == 0 || kind != CK_FANOUT)
                continue;
            const uint64_t d0 = (reinterpret_cast<uintptr_t>(dsts[0]) + seg_dst[s] - seg_src[s]) % kVecBytes;
            for (int q = 1; q < ndst; ++q)
                shifted = shifted && (reinterpret_cast<uintptr_t>(dsts[q]) + seg_dst[s] - seg_src[s]) % kVecBytes == d0;
        }
        vec = shifted;
    }
    a.shifted = shifted ? 1 : 0;
    p->vec = vec ? 1 : 0;
    p->U = vec ? pick_u_copy(kind, nseg, c.stages) : 1;
    // 64-lane tiles over 256-lane ones, cold with streaming stores on
    // MI355X: +2 % on the exchange (AllToAllV, 2 slots per lane) and +2 % on
    // the fan-out (AllGather, 1 slot), whose tiles write P times what they
    // read. A flat copy of 256 MiB with
    // streaming stores, cold on MI355X: 128 lanes x 2 slots (4 KiB tiles)
    // 6.33 TB/s, 256 x 2 6.25, 256 x 4 5.70, and 1 KiB tiles 4.7 (the
    // workgroup dispatch rate bounds a grid of that many small tiles).
    p->wg = !vec ? 256 : (nseg > 1 ? 64 : 128);
    // The shifted path, measured on MI355X: the fan-out best at 256 lanes x
    // 1 slot (Zipf AllGatherV of 8 x 64 MiB in single-element partitions:
    // 5.79 TB/s, 5.71 at 64 x 1, 4.8-5.4 deeper), the exchange at 128 x 2
    // (AllToAllV of 8 x 4096 rows of 7167 bf16: 5.89 TB/s, 5.73 at 64 x 2,
    // 3.5-3.7 with one slot).
    if (shifted && nseg > 1) {
        p->wg = kind == CK_FANOUT ? 256 : 128;
        if (!c.stages)
            p->U = kind == CK_FANOUT ? 1 : 2;
    }
    int64_t bytes = 0;
    for (int s = 0; s < nseg; ++s)
        bytes += cnt[s] * row_bytes;
    if (bytes < kSmallSlots * kVecBytes && !c.stages) {
        p->U = 1;                 // latency path, as for the reduce family
        p->wg = 64;
    }
    if (c.lanes)
        p->wg = c.lanes;
    // A fan-out beyond the latency path runs in blocked order
    // (k_copy_fan_blocked): one output at a time per block, the block's
    // source re-read from each XCD's L2. Measured on MI355X (1 -> 8 fan-out
    // of 256 MiB, cold): 8 KiB tiles (256 lanes x 2 slots) and 4-16 MiB
    // blocks write at 6.7-6.9 TB/s, against 5.2 TB/s for one load feeding 8
    // stores; 64 MiB blocks (8 MiB per XCD, beyond its 4 MB L2) fall to 4.1.
    // In the AllGather of 8 x 64 MiB: 256 x 2 with 8 MiB blocks 6.03 TB/s,
    // 4 and 16 MiB 5.95, 256 x 4 5.6-5.7, 256 x 8 4.8-5.3.
    const bool blocked = vec && !shifted && kind == CK_FANOUT && ndst > 1 && nseg <= kMaxRanks &&
                         bytes >= kSmallSlots * kVecBytes && !(c.flags & ATOM_F_XCD_ORDER);
    if (blocked) {
        if (!c.lanes)
            p->wg = 256;
        if (!c.stages)
            p->U = 2;
    }
    a.tile_bytes = static_cast<int64_t>(p->wg) * p->U * kVecBytes;   // a power of two (seg_tile_shift)
    // Aligned tiles pay off for the fan-out; the exchange moves one byte out
    // per byte in, and aligning its destination misaligns its source, so it
    // keeps segment-relative tiles. Measured on MI355X, cold with streaming
    // stores: the AllGatherV of 8 x 64 MiB in Zipf(0.125) partitions 5.53
    // TB/s aligned against 4.47 unaligned; the AllToAllV of 8 x 4096 x 7168
    // 6.22 segment-relative against 5.35 aligned.
    a.align = (vec && kind == CK_FANOUT) ? 1 : 0;
    int64_t t = 0;
    for (int s = 0; s < nseg; ++s) {
        a.cnt[s] = static_cast<int32_t>(cnt[s]);
        a.seg_tile_begin[s] = static_cast<int32_t>(t);
        const int64_t h = a.head[s];
        // Fan-out vector path: tiles start at addresses aligned to the tile
        // size in the destination (P stores per load: the side with the most
        // bytes), counted from the segment's first 16-byte boundary.
        int64_t shift = 0;
        if (a.align)
            shift = seg_tile_shift(reinterpret_cast<uintptr_t>(dsts[0]) + seg_dst[s] + h, a.tile_bytes);
        const int64_t rest = cnt[s] * row_bytes - h;
        int64_t tiles = rest ? ceil_div(rest + shift, a.tile_bytes) : 0;
        if (h > 0 && tiles == 0)
            tiles = 1;                   // a segment that is all head still needs its tile
        if (shifted && rest > 0) {
            // the segment's source vectors, plus one for the last slot, from
            // the vector that starts a tile at the source (exchange) or at
            // output 0 (fan-out), as k_copy_shift places them
            const int64_t tv = static_cast<int64_t>(p->wg) * p->U;
            const int64_t vlo = static_cast<int64_t>(seg_src[s] / kVecBytes);
            int64_t v0 = vlo & ~(tv - 1);
            if (a.align) {
                const int64_t m0 = static_cast<int64_t>(reinterpret_cast<uintptr_t>(dsts[0]) + seg_dst[s] - seg_src[s]);
                v0 = vlo - ((vlo + (m0 >> 4)) & (tv - 1));
            }
            const int64_t nv = static_cast<int64_t>((seg_src[s] + rest - 1) / kVecBytes) + 2 - v0;
            tiles = ceil_div(nv, tv);
        }
        t += tiles;
    }
    a.seg_tile_begin[nseg] = static_cast<int32_t>(t);
    a.ntiles = t;
    a.row_bytes = row_bytes;
    a.kind = kind;
    a.P = P;
    a.nseg = nseg;
    a.ndst = ndst;
    a.esize = esize;
    // Streaming stores except on the latency path (as for the reduce family).
    a.nt_store = ((c.flags & ATOM_F_NO_NT) || bytes < kSmallSlots * kVecBytes) ? 0 : 1;
    a.xcd_remap = (c.flags & ATOM_F_XCD_ORDER) ? 1 : 0;
    p->grid = pick_grid(t, c.num_wgs);
    p->exec = t > 0 ? EX_COPY : EX_NONE;
    a.block_shift = -1;
    if (blocked && t > 0) {
        // Blocks of a power of two of tiles, at least the 8 XCDs; one
        // workgroup per task (a grid stride only beyond kMaxGridBlocked, or
        // for a caller's num_wgs), so workgroup w is task w.
        int32_t lb = 3;
        while ((a.tile_bytes << (lb + 1)) <= kFanBlockBytes)
            ++lb;
        a.block_shift = lb;
        a.nwork = ceil_div(t, int64_t(1) << lb) * (int64_t(1) << lb) * ndst;
        int64_t off = 0;
        for (int s = 0; s < nseg; ++s) {
            a.seg_off[s] = off;
            off += cnt[s] * row_bytes;
        }
        a.seg_off[nseg] = off;
        p->grid = std::max<int64_t>(1, std::min(a.nwork, c.num_wgs > 0 ? c.num_wgs : kMaxGridBlocked));
    }
    // Uniform form of the latency path (as for the reduce family): equal
    // segments, no heads, the same tile count each, one tile per workgroup;
    // the grid is tiles-per-segment x segments.
    a.grid_segs = 0;
    const int64_t tps = nseg > 0 ? a.seg_tile_begin[1] : 0;
    bool uniform = vec && !shifted && t > 0 && bytes < kSmallSlots * kVecBytes && !a.xcd_remap &&
                   c.num_wgs == 0 && nseg <= 65535;
    for (int s = 0; s < nseg && uniform; ++s)
        uniform = cnt[s] == cnt[0] && a.head[s] == 0 && a.seg_tile_begin[s] == s * tps;
    if (uniform) {
        a.grid_segs = nseg;
        p->grid = tps;
    }
}

// Limit that keeps per-segment tile indices in 32 bits.
constexpr int64_t kMaxTiles = INT32_MAX;

// SNAC launch over a segment list (kargs.hpp: SnacKind). cnt[s] rows of rb
// bytes per segment. max_ring_bytes > 0 bounds the ring (the fixed
// workspace of atom_collective_noalloc): without a caller's ring depth the
// depth is cut to fit, a caller's depth or chunk that does not fit is
// ATOM_ERR_LIMIT.
atom_status build_snac(Plan* p, int32_t sk, int P, void* const* ins, void* const* outs,
                       const int64_t* cnt, int nseg, int64_t rb, const Cfg& c,
                       int64_t max_ring_bytes)
{
    SnacArgs& a = p->sa;
    std::memset(&a, 0, sizeof a);
    const bool reduce = sk == SK_SCATTER || sk == SK_ALLRED;
    // Segment geometry, as the kernel derives it: bytes, source offset (of
    // the segment's own source, or of every source for a reduce) and
    // destination offset. A segment whose streams all sit at one offset d
    // from 16-byte alignment takes the vector path (for d > 0 its pieces are
    // staged 112 + d bytes into their ring place, so ring, source and
    // destination share their 16-byte phase and the staged body starts on a
    // 128-byte line; each piece's two ends move element by element);
    // otherwise it is staged element by element. Measured on MI355X with
    // every buffer one bf16 element off: the staged AllGather of 8 x 64 MiB
    // 2.40 TB/s element by element, 4.99 on this path (5.16 aligned).
    int64_t bytes[kMaxSegs], total = 0, largest = 0;
    int64_t col_rows[kMaxRanks] = {}, run_rows = 0;
    for (int r = 0; r < P; ++r) {
        a.src[r] = ins[r];
        a.dst[r] = outs[r];
    }
    for (int s = 0; s < nseg; ++s) {
        bytes[s] = cnt[s] * rb;
        total += bytes[s];
        largest = std::max(largest, bytes[s]);
        a.cnt[s] = static_cast<int32_t>(cnt[s]);
        // Offset from 16-byte alignment of every stream of the segment at
        // its first byte. All equal (d): the vector path, staged d bytes
        // past a 16-byte boundary, with element-wise heads and tails when
        // d > 0. Sources equal (d) and some destination not: staged the
        // same way, consumed by the shifted path. Sources unequal:
        // element-wise.
        int src_d = -1, dst_d = -1;
        bool src_same = true, all_same = true;
        auto mis = [](const void* b, int64_t off) {
            return static_cast<int>((reinterpret_cast<uintptr_t>(b) + static_cast<uint64_t>(off)) % kVecBytes);
        };
        auto at_src = [&](const void* b, int64_t off) {
            const int m = mis(b, off);
            if (src_d < 0)
                src_d = m;
            src_same = src_same && m == src_d;
        };
        auto at_dst = [&](const void* b, int64_t off) {
            const int m = mis(b, off);
            if (dst_d < 0)
                dst_d = m;
            all_same = all_same && m == dst_d;
        };
        if (sk == SK_EXCHANGE) {
            const int r = s / P, j = s % P;
            int64_t src_rows = 0;
            for (int jj = 0; jj < j; ++jj)
                src_rows += cnt[r * P + jj];
            at_src(ins[r], src_rows * rb);
            at_dst(outs[j], col_rows[j] * rb);
            col_rows[j] += cnt[s];
        } else {
            const int64_t off = run_rows * rb;
            if (sk == SK_GATHER) {
                at_src(ins[s], 0);
            } else {
                for (int r = 0; r < P; ++r)
                    at_src(ins[r], off);
            }
            if (sk == SK_SCATTER) {
                at_dst(outs[s], 0);
            } else {
                for (int q = 0; q < P; ++q)
                    at_dst(outs[q], off);
            }
            run_rows += cnt[s];
        }
        all_same = all_same && src_same && src_d == dst_d;
        a.elem[s] = static_cast<uint8_t>(all_same ? SE_VEC : (src_same ? SE_SHIFT : SE_ELEM));
        a.head[s] = static_cast<uint8_t>(src_same ? src_d : 0);
    }
    if (total == 0)
        return ATOM_OK;
    // Chunk: the caller's, else the one measured best on MI355X for the
    // stage (a copying stage 512 KiB, 2 MiB once its largest segment reaches
    // 256 MiB; a reducing one 2 MiB: all in the 512 KiB - 2 MiB range of
    // Table 3's bandwidth-delay rule). The staged AllGather, 512 KiB / 2 MiB
    // chunks: 8 x 64 MiB 0.924 / 0.926 ms cold; 8 x 1 GiB 13.77 / 13.72 ms
    // cold and 13.95 / 13.69 ms in a warm size sweep; 8 x 256 MiB 3.51 /
    // 3.44 ms warm.
    int64_t chunk = c.chunk_set ? c.chunk
                    : reduce    ? kDefaultChunkAllReduce
                    : largest >= kHugeCopySegment ? kHugeCopyChunk
                                                  : kDefaultChunkAllGather;
    // Piece (the task granule): the caller's, else the largest power of two
    // from 8 KiB to 64 KiB (32 KiB for a copying stage) that still gives
    // about one persistent grid's worth of staging tasks (total / piece >=
    // 2 * 512), so a medium message is spread over many workgroups instead
    // of a few (smaller pieces cost more in hand-offs than they gain).
    // Measured cold on MI355X with 512 lanes and the half-depth lead: the
    // staged AllGather of 8 x 64 MiB 0.964 ms with 64 KiB pieces, 0.922-0.925
    // with 32 KiB (16 KiB: 1.00), of 8 x 1 GiB 14.46 -> 13.73 ms; the
    // composed AllReduce and the ReduceScatterV keep 64 KiB (32 KiB 1-3 %
    // slower: a reducing piece reads P inputs, so it is already P times the
    // work).
    int64_t piece = c.piece;
    if (!piece) {
        const int64_t top = reduce ? kPieceBytes : kCopyPieceBytes;
        piece = kMinAutoPiece;
        while (piece < top && total / (2 * piece) >= kSnacGrid)
            piece *= 2;
    }
    piece = std::min(piece, chunk);
    // A largest segment smaller than the chunk: one chunk of just enough
    // whole pieces, so no task handles an empty piece.
    if (largest < chunk)
        chunk = std::max<int64_t>(1, ceil_div(largest, piece)) * piece;
    if (max_ring_bytes > 0 && chunk > max_ring_bytes)
        return ATOM_ERR_LIMIT;
    int64_t q = 0, per0 = -1;
    bool same = true;
    for (int s = 0; s < nseg; ++s) {
        a.chunk_begin[s] = static_cast<int32_t>(q);
        const int64_t nc = ceil_div(bytes[s], chunk);
        same = same && (per0 < 0 || nc == per0);
        per0 = nc;
        q += nc;
        if (q > INT32_MAX)
            return ATOM_ERR_INVALID_ARG;
    }
    a.chunk_begin[nseg] = static_cast<int32_t>(q);
    // Equal chunk counts (the uniform collectives): chunk q belongs to
    // segment q % nseg, so the producers stream from every source at once.
    a.interleave = same ? 1 : 0;
    a.kind = sk;
    a.P = P;
    a.nseg = nseg;
    a.row_bytes = rb;
    a.chunk_bytes = chunk;
    a.piece_bytes = piece;
    a.pieces = static_cast<int32_t>(chunk / piece);
    a.slots = c.slots;
    if (!c.slots_set) {
        // Table 3's rule applied to one device: the ring holds at least one
        // bandwidth-delay product of HBM (8 TB/s) times the cross-XCD
        // stage-notify-consume round trip (~4 us measured), about 32 MiB.
        const int64_t want = ceil_div(kSnacInflightBytes, chunk);
        a.slots = static_cast<int32_t>(std::max<int64_t>(kDefaultSlots, std::min<int64_t>(kMaxSlots, want)));
        if (max_ring_bytes > 0)
            a.slots = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(a.slots, max_ring_bytes / chunk)));
    } else if (max_ring_bytes > 0 && chunk * a.slots > max_ring_bytes) {
        return ATOM_ERR_LIMIT;
    }
    // Lead (chunks staged before the first consumer in the ticket order):
    // the caller's, else half the ring depth. With the full depth a
    // producer waits for the consumers of its slot, claimed just before it
    // (per-task clock stamps on MI355X: 21-37 % of all workgroup time); half
    // the depth leaves those slots free. Measured cold on MI355X over leads
    // D..D/8: the Zipf ReduceScatterV of 8 x 256 MiB (a reducing producer is
    // the long task) 0.547-0.570 -> 0.486-0.495 ms, the composed AllReduce
    // 0.818 -> 0.811 ms, the AllGather of 8 x 1 GiB 14.95 -> 14.42 ms; the
    // other copying rows moved by -2..+2 % between runs.
    a.lead = c.lead ? std::min(c.lead, a.slots) : std::max(1, a.slots / 2);
    a.trace = c.trace;
    a.nchunks = q;
    // A slot's count word holds the pieces of every chunk the slot takes in
    // 32 bits each (staged, consumed).
    if (ceil_div(q, a.slots) * a.pieces >= (int64_t(1) << 32))
        return ATOM_ERR_LIMIT;
    a.ntasks = 2 * a.nchunks * a.pieces;
    a.dtype = p->dtype;
    a.nt_store = (c.flags & ATOM_F_NO_NT) ? 0 : 1;
    a.wait_ticks = c.wait_us;             // converted to clock ticks at launch
    a.jitter_ticks = c.jitter_us;         // likewise
    a.jitter_seed = c.jitter_seed;
    bool any_elem = false, any_shift = false;
    for (int s = 0; s < nseg; ++s) {
        any_elem = any_elem || (a.elem[s] == SE_ELEM && bytes[s] > 0);
        any_shift = any_shift || (a.elem[s] == SE_SHIFT && bytes[s] > 0);
    }
    p->vec = any_elem ? 0 : 1;
    p->snac_shifted = any_shift ? 1 : 0;
    // Lanes per workgroup: 512 (two persistent workgroups of 8 waves per
    // CU). Measured on MI355X with streaming output stores: the composed
    // AllReduce, whose reducing stage reads P inputs per staged byte, +5 %
    // over 256 lanes; the AllGather of 8 x 64 MiB +2 %.
    p->wg = c.lanes ? c.lanes : 512;
    // 16-byte slots per lane in flight: 8 measured best for the staged
    // AllGather (+10% over 4); a reducing stage's depths are fixed by its
    // kernel (2 while reducing P <= 8 inputs, 8 while consuming).
    p->U = c.stages ? c.stages : 8;
    p->slots = a.slots;
    p->chunk_bytes = chunk;
    a.slot_bytes = chunk + kSlotPad;
    p->ring_bytes = a.slot_bytes * a.slots;
    // Workgroups: the caller's, else one per staged piece the ring can hold
    // (slots * pieces per chunk), at most 512. A larger grid than the ring's
    // window only adds waiting workgroups: measured 5-18 % slower when the
    // window is smaller than the grid.
    const int64_t window = static_cast<int64_t>(a.slots) * a.pieces;
    p->grid = std::max<int64_t>(
        1, std::min<int64_t>(a.ntasks, c.num_wgs ? c.num_wgs : std::min(kSnacGrid, window)));
    // Small calls (at most kSnacStaticTasks tasks, one workgroup each, no
    // caller grid) skip the ticket: workgroup b runs task b. Dispatch in
    // index order puts every task's producers (smaller tickets) on the chip
    // first, and a grid this small fits the chip at once; the waits stay
    // bounded either way. Saves the ticket atomic's round trip before the
    // first task and after the last.
    a.static_tasks = (!c.num_wgs && p->grid == a.ntasks && a.ntasks <= kSnacStaticTasks) ? 1 : 0;
    // A call whose ring holds every chunk (no slot is reused), each of whose
    // segments has every stream at one offset from 16-byte alignment (the
    // vector path, SE_VEC) and whose staged bytes fit the tagged ring hands
    // off through tagged words (k_snac_tagged): the notify
    // travels in the staged words' tags, the producer neither waits for its
    // stores to complete nor counts, and the consumer holds its words as it
    // sees them instead of reading the ring after a count. One workgroup
    // per task, task = blockIdx.x: producers never wait, and a consumer
    // waits only for producers with smaller indices, which the in-order
    // dispatch has started before it, so the grid need not fit the chip.
    // Measured on MI355X (event-timed, staged AllGather): 256 KiB, 512 KiB
    // and 1 MiB per rank 19.5, 23.4 and 26.9 us through the ticket and the
    // counts. A staged word takes 8 bytes on the tagged ring instead of 4,
    // so larger calls keep the counts: tagged / counted, AllGather of 8 x 2
    // MiB (16 MiB staged) 41.3 / 44.8 us, of 8 x 4 MiB 77.6 / 72.2 us;
    // AllReduce of 16 MiB 58.1 / 62.4 us, of 32 MiB 132.7 / 122.1 us.
    // A segment whose streams share an offset d from 16-byte alignment is
    // staged in the aligned vectors enclosing each piece: one vector more
    // than the piece at most, so its place gets one more group of 64.
    bool tag_ok = !c.num_wgs && !(c.flags & ATOM_F_COUNTED) && q <= a.slots && piece % 1024 == 0 &&
                  chunk % piece == 0;
    bool off = false;
    for (int s = 0; s < nseg && tag_ok; ++s) {
        tag_ok = bytes[s] == 0 || a.elem[s] == SE_VEC;
        off = off || (bytes[s] > 0 && a.head[s] != 0);
    }
    a.tag_place = 4 * (piece / kVecBytes + (off ? 64 : 0));
    tag_ok = tag_ok && q * (chunk / piece) * a.tag_place * 8 <= kTagBytes;
    a.tagged = tag_ok ? 1 : 0;
    if (tag_ok) {
        p->grid = a.ntasks;
        a.static_tasks = 1;
    }
    p->exec = reduce ? EX_SNAC_REDUCE : EX_SNAC_COPY;
    return ATOM_OK;
}

}  // namespace

// --------------------------------------------------------------------------

atom_status plan_copy(void* dst, const void* src, size_t bytes, const atom_config* cfg, Plan* p)
{
    Cfg c;
    atom_status st = read_cfg(cfg, &c);
    if (st != ATOM_OK)
        return st;
    if (bytes > static_cast<size_t>(INT64_MAX / 2))
        return ATOM_ERR_INVALID_ARG;
    const int64_t b = static_cast<int64_t>(bytes);
    if (b > 0 && (dst == nullptr || src == nullptr))
        return ATOM_ERR_INVALID_ARG;
    Range ri = range_of(src, b), ro = range_of(dst, b);
    if (!disjoint(&ri, 1, &ro, 1))
        return ATOM_ERR_INVALID_ARG;
    if (c.flags & ATOM_F_STAGED)
        return ATOM_ERR_UNSUPPORTED;
    p->reset();
    p->kind = ATOM_COLL_NONE;
    p->P = 1;
    uintptr_t bits = reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src) |
                     static_cast<uintptr_t>(b);
    int es = (bits & 3) == 0 ? 4 : ((bits & 1) == 0 ? 2 : 1);
    p->esize = es;
    p->in_elems = b;
    p->out_elems[0] = b;
    p->credited_bytes = 2 * b;
    if (b == 0)
        return ATOM_OK;
    if (ceil_div(b, 256 * kVecBytes) > kMaxTiles)
        return ATOM_ERR_INVALID_ARG;
    const void* srcs[1] = {src};
    void* dsts[1] = {dst};
    int64_t one = 1;
    build_copy(p, CK_FANOUT, 1, srcs, 1, dsts, 1, &one, 1, b, es, c);
    return ATOM_OK;
}

atom_status plan_reduce(void* dst, const void* const* srcs, int32_t nsrcs, int64_t count,
                        atom_dtype dtype, atom_op op, const atom_config* cfg, Plan* p)
{
    Cfg c;
    atom_status st = read_cfg(cfg, &c);
    if (st != ATOM_OK)
        return st;
    const int es = esize_of(dtype);
    if (es == 0 || srcs == nullptr || nsrcs < 1 || nsrcs > kMaxRanks || count < 0)
        return ATOM_ERR_INVALID_ARG;
    if (op != ATOM_OP_SUM && op != ATOM_OP_COPY)
        return ATOM_ERR_INVALID_ARG;
    if (op == ATOM_OP_COPY && nsrcs != 1)
        return ATOM_ERR_UNSUPPORTED;
    if (c.flags & ATOM_F_STAGED)
        return ATOM_ERR_UNSUPPORTED;
    int64_t bytes;
    if (!mul_ok(count, es, &bytes))
        return ATOM_ERR_INVALID_ARG;
    Range ins[kMaxRanks];
    for (int r = 0; r < nsrcs; ++r) {
        if (!buffer_ok(srcs[r], bytes, es))
            return ATOM_ERR_INVALID_ARG;
        ins[r] = range_of(srcs[r], bytes);
    }
    if (!buffer_ok(dst, bytes, es))
        return ATOM_ERR_INVALID_ARG;
    Range ro = range_of(dst, bytes);
    if (!disjoint(ins, nsrcs, &ro, 1))
        return ATOM_ERR_INVALID_ARG;
    p->reset();
    p->kind = ATOM_COLL_NONE;
    p->dtype = dtype == ATOM_DT_BF16 ? DT_BF16 : DT_F32;
    p->esize = es;
    p->P = nsrcs;
    p->in_elems = count;
    p->out_elems[0] = count;
    p->credited_bytes = (static_cast<int64_t>(nsrcs) + 1) * bytes;
    if (count == 0)
        return ATOM_OK;
    int64_t off[2] = {0, count};
    void* dsts[1] = {dst};
    build_reduce(p, nsrcs, srcs, 1, dsts, 1, off, RM_SCATTER, c);
    return ATOM_OK;
}

atom_status plan_collective_ex(const atom_layout* in, const atom_layout* out, atom_op op,
                               const atom_config* cfg, int64_t max_ring_bytes, Plan* p)
{
    Cfg c;
    atom_status st = read_cfg(cfg, &c);
    if (st != ATOM_OK)
        return st;
    if (!in || !out)
        return ATOM_ERR_INVALID_ARG;
    const int P = in->nranks;
    if (P < 1 || P > kMaxRanks || out->nranks != P)
        return ATOM_ERR_INVALID_ARG;
    if (!in->bufs || !out->bufs)
        return ATOM_ERR_INVALID_ARG;
    const int es = esize_of(in->dtype);
    if (es == 0 || out->dtype != in->dtype)
        return ATOM_ERR_INVALID_ARG;
    if (op != ATOM_OP_COPY && op != ATOM_OP_SUM)
        return ATOM_ERR_INVALID_ARG;
    auto kind_ok = [](atom_layout_kind k) {
        return k == ATOM_LAYOUT_PARTITIONED || k == ATOM_LAYOUT_SHARD ||
               k == ATOM_LAYOUT_GATHERED || k == ATOM_LAYOUT_TRANSPOSED;
    };
    if (!kind_ok(in->kind) || !kind_ok(out->kind))
        return ATOM_ERR_INVALID_ARG;

    // ---- which collective does the naming describe?
    const bool v = in->counts != nullptr;
    atom_collective_kind kind = ATOM_COLL_NONE;
    if (in->kind == ATOM_LAYOUT_PARTITIONED && out->kind == ATOM_LAYOUT_SHARD && op == ATOM_OP_SUM)
        kind = v ? ATOM_COLL_REDUCE_SCATTER_V : ATOM_COLL_REDUCE_SCATTER;
    else if (in->kind == ATOM_LAYOUT_SHARD && out->kind == ATOM_LAYOUT_GATHERED && op == ATOM_OP_COPY)
        kind = v ? ATOM_COLL_ALL_GATHER_V : ATOM_COLL_ALL_GATHER;
    else if (in->kind == ATOM_LAYOUT_PARTITIONED && out->kind == ATOM_LAYOUT_TRANSPOSED &&
             op == ATOM_OP_COPY)
        kind = v ? ATOM_COLL_ALL_TO_ALL_V : ATOM_COLL_ALL_TO_ALL;
    else if (in->kind == ATOM_LAYOUT_PARTITIONED && out->kind == ATOM_LAYOUT_GATHERED &&
             op == ATOM_OP_SUM && !v)
        kind = ATOM_COLL_ALL_REDUCE;
    if (kind == ATOM_COLL_NONE)
        return ATOM_ERR_UNSUPPORTED;

    // ---- counts (V variants) or the uniform partition size
    const int ncnt = (kind == ATOM_COLL_ALL_TO_ALL_V) ? P * P : P;
    int64_t cnt[kMaxSegs];
    int64_t row = 1;
    int64_t n = 0;
    if (v) {
        if (in->row_elems < 1 || out->row_elems != in->row_elems)
            return ATOM_ERR_INVALID_ARG;
        row = in->row_elems;
        for (int e = 0; e < ncnt; ++e) {
            cnt[e] = in->counts[e];
            if (cnt[e] < 0 || cnt[e] > INT32_MAX)
                return ATOM_ERR_INVALID_ARG;
            if (out->counts && out->counts[e] != cnt[e])
                return ATOM_ERR_INVALID_ARG;
        }
    } else {
        if (out->counts)
            return ATOM_ERR_INVALID_ARG;
        n = in->part_elems;
        if (n < 0 || out->part_elems != n)
            return ATOM_ERR_INVALID_ARG;
    }
    int64_t row_bytes;
    if (!mul_ok(row, es, &row_bytes))
        return ATOM_ERR_INVALID_ARG;

    // ---- per-buffer element counts
    int64_t in_el[kMaxRanks], out_el[kMaxRanks];
    int64_t total = 0;   // elements of one "P*n" index space (per rank)
    if (!v) {
        if (!mul_ok(n, P, &total))
            return ATOM_ERR_INVALID_ARG;
    }
    int64_t tmp;
    switch (kind) {
    case ATOM_COLL_REDUCE_SCATTER:
        for (int r = 0; r < P; ++r) { in_el[r] = total; out_el[r] = n; }
        break;
    case ATOM_COLL_ALL_GATHER:
        for (int r = 0; r < P; ++r) { in_el[r] = n; out_el[r] = total; }
        break;
    case ATOM_COLL_ALL_TO_ALL:
    case ATOM_COLL_ALL_REDUCE:
        for (int r = 0; r < P; ++r) { in_el[r] = total; out_el[r] = total; }
        break;
    case ATOM_COLL_REDUCE_SCATTER_V:
    case ATOM_COLL_ALL_GATHER_V: {
        int64_t rows = 0;
        for (int k = 0; k < P; ++k)
            rows += cnt[k];
        if (!mul_ok(rows, row, &total))
            return ATOM_ERR_INVALID_ARG;
        for (int k = 0; k < P; ++k) {
            if (!mul_ok(cnt[k], row, &tmp))
                return ATOM_ERR_INVALID_ARG;
            if (kind == ATOM_COLL_REDUCE_SCATTER_V) { in_el[k] = total; out_el[k] = tmp; }
            else { in_el[k] = tmp; out_el[k] = total; }
        }
        break;
    }
    case ATOM_COLL_ALL_TO_ALL_V:
        for (int r = 0; r < P; ++r) {
            int64_t send = 0, recv = 0;
            for (int j = 0; j < P; ++j) {
                send += cnt[r * P + j];
                recv += cnt[j * P + r];
            }
            if (!mul_ok(send, row, &in_el[r]) || !mul_ok(recv, row, &out_el[r]))
                return ATOM_ERR_INVALID_ARG;
        }
        break;
    default:
        return ATOM_ERR_UNSUPPORTED;
    }

    // ---- buffers: element-aligned, non-NULL unless empty, outputs disjoint
    Range ri[kMaxRanks], ro[kMaxRanks];
    int64_t in_bytes_total = 0, out_bytes_total = 0;
    for (int r = 0; r < P; ++r) {
        int64_t bi, bo;
        if (!mul_ok(in_el[r], es, &bi) || !mul_ok(out_el[r], es, &bo))
            return ATOM_ERR_INVALID_ARG;
        if (!buffer_ok(in->bufs[r], bi, es) || !buffer_ok(out->bufs[r], bo, es))
            return ATOM_ERR_INVALID_ARG;
        ri[r] = range_of(in->bufs[r], bi);
        ro[r] = range_of(out->bufs[r], bo);
        in_bytes_total += bi;
        out_bytes_total += bo;
        if (in_bytes_total < 0 || out_bytes_total < 0)
            return ATOM_ERR_INVALID_ARG;
    }
    if (!disjoint(ri, P, ro, P))
        return ATOM_ERR_INVALID_ARG;

    const bool staged = (c.flags & ATOM_F_STAGED) != 0;

    p->reset();
    p->kind = kind;
    p->dtype = in->dtype == ATOM_DT_BF16 ? DT_BF16 : DT_F32;
    p->esize = es;
    p->P = P;
    p->in_elems = in_el[0];
    for (int r = 0; r < P; ++r)
        p->out_elems[r] = out_el[r];

    // Credited (algorithmic) bytes: every input element read once, every
    // output element written once; a reduced element counts its P reads.
    switch (kind) {
    case ATOM_COLL_REDUCE_SCATTER:
    case ATOM_COLL_REDUCE_SCATTER_V:
        p->credited_bytes = static_cast<int64_t>(P + 1) * total * es;
        break;
    case ATOM_COLL_ALL_REDUCE:
        p->credited_bytes = 2 * static_cast<int64_t>(P) * total * es;
        break;
    case ATOM_COLL_ALL_GATHER:
    case ATOM_COLL_ALL_GATHER_V:
        p->credited_bytes = static_cast<int64_t>(1 + P) * total * es;
        break;
    default:
        p->credited_bytes = in_bytes_total + out_bytes_total;
        break;
    }
    if (in_bytes_total == 0 && out_bytes_total == 0)
        return ATOM_OK;

    // ---- the launch
    int64_t ones[kMaxSegs];
    for (int e = 0; e < kMaxSegs; ++e)
        ones[e] = 1;
    const int64_t rb = v ? row_bytes : n * es;           // bytes per counted row
    if (staged) {
        // Every collective runs through SNAC as a list of segments derived
        // from its layouts (the abstract: one orchestration for all of them).
        const bool a2a = kind == ATOM_COLL_ALL_TO_ALL || kind == ATOM_COLL_ALL_TO_ALL_V;
        int32_t sk = SK_GATHER;
        if (a2a)
            sk = SK_EXCHANGE;
        else if (kind == ATOM_COLL_REDUCE_SCATTER || kind == ATOM_COLL_REDUCE_SCATTER_V)
            sk = SK_SCATTER;
        else if (kind == ATOM_COLL_ALL_REDUCE)
            sk = SK_ALLRED;
        return build_snac(p, sk, P, in->bufs, out->bufs, v ? cnt : ones, a2a ? P * P : P, rb, c,
                          max_ring_bytes);
    }
    int64_t off[kMaxRanks + 1];
    switch (kind) {
    case ATOM_COLL_REDUCE_SCATTER:
    case ATOM_COLL_REDUCE_SCATTER_V: {
        off[0] = 0;
        for (int k = 0; k < P; ++k)
            off[k + 1] = off[k] + (v ? cnt[k] * row : n);
        build_reduce(p, P, in->bufs, P, out->bufs, P, off, RM_SCATTER, c);
        break;
    }
    case ATOM_COLL_ALL_REDUCE: {
        off[0] = 0;
        off[1] = total;
        build_reduce(p, P, in->bufs, P, out->bufs, 1, off, RM_FANOUT, c);
        break;
    }
    case ATOM_COLL_ALL_GATHER:
    case ATOM_COLL_ALL_GATHER_V: {
        if (ceil_div(total * es, 256 * kVecBytes) > kMaxTiles)
            return ATOM_ERR_INVALID_ARG;
        build_copy(p, CK_FANOUT, P, in->bufs, P, out->bufs, P, v ? cnt : ones, P, rb, es, c);
        break;
    }
    case ATOM_COLL_ALL_TO_ALL:
    case ATOM_COLL_ALL_TO_ALL_V: {
        if (ceil_div(in_bytes_total, 256 * kVecBytes) + P * P > kMaxTiles)
            return ATOM_ERR_INVALID_ARG;
        build_copy(p, CK_EXCHANGE, P, in->bufs, P, out->bufs, P, v ? cnt : ones, P * P, rb, es, c);
        break;
    }
    default:
        return ATOM_ERR_UNSUPPORTED;
    }
    return ATOM_OK;
}

atom_status plan_collective(const atom_layout* in, const atom_layout* out, atom_op op,
                            const atom_config* cfg, Plan* p)
{
    return plan_collective_ex(in, out, op, cfg, 0, p);
}

// ---- MoE (Table 2, expert parallelism) ----------------------------------

namespace {

// The routing fields every MoE call needs; T*k entries per rank.
atom_status check_routing(const atom_moe_routing* rt)
{
    if (!rt || rt->reserved != 0)
        return ATOM_ERR_INVALID_ARG;
    const int64_t P = rt->nranks, E = rt->num_experts, k = rt->topk, T = rt->tokens;
    if (P < 1 || P > kMaxRanks || E < P || E > ATOM_MOE_MAX_EXPERTS || E % P != 0 || k < 1 ||
        k > kMoeMaxTopk || T < 0 || T > ATOM_MOE_MAX_ENTRIES || T * k > ATOM_MOE_MAX_ENTRIES)
        return ATOM_ERR_INVALID_ARG;
    if (T > 0) {
        if (!rt->expert_ids || !rt->positions)
            return ATOM_ERR_INVALID_ARG;
        for (int r = 0; r < P; ++r)
            if (!buffer_ok(rt->expert_ids[r], T * k * 4, 4) || !buffer_ok(rt->positions[r], T * k * 4, 4))
                return ATOM_ERR_INVALID_ARG;
    }
    return ATOM_OK;
}

int32_t moe_chunks(int64_t n) { return static_cast<int32_t>(std::max<int64_t>(1, ceil_div(n, kMoeChunk))); }

}  // namespace

int64_t moe_scratch_bytes(int32_t P, int32_t E, int32_t k, int64_t T)
{
    if (P < 1 || P > kMaxRanks || E < P || E > ATOM_MOE_MAX_EXPERTS || E % P != 0 || k < 1 ||
        k > kMoeMaxTopk || T < 0 || T > ATOM_MOE_MAX_ENTRIES || T * k > ATOM_MOE_MAX_ENTRIES)
        return 0;
    const int64_t ints = static_cast<int64_t>(P) * moe_chunks(T * k) * E;
    return ceil_div(ints * 4, 256) * 256;
}

atom_status plan_moe_route(const atom_moe_routing* rt, MoeRoutePlan* p)
{
    if (!p)
        return ATOM_ERR_INVALID_ARG;
    if (atom_status st = check_routing(rt); st != ATOM_OK)
        return st;
    const int P = rt->nranks, E = rt->num_experts;
    const int64_t n = rt->tokens * rt->topk;
    if (!rt->counts || !rt->recv_rows || !rt->scratch || !aligned(rt->scratch, 16) ||
        !aligned(rt->counts, 4) || !aligned(rt->recv_rows, 8))
        return ATOM_ERR_INVALID_ARG;
    const int64_t sbytes = moe_scratch_bytes(P, E, rt->topk, rt->tokens);
    // Written ranges (positions, counts, recv, scratch) must be disjoint from
    // each other and from the ids.
    Range ins[kMaxRanks], outs[kMaxRanks + 3];
    int nin = 0, nout = 0;
    for (int r = 0; r < P && n > 0; ++r) {
        ins[nin++] = range_of(rt->expert_ids[r], n * 4);
        outs[nout++] = range_of(rt->positions[r], n * 4);
    }
    outs[nout++] = range_of(rt->counts, static_cast<int64_t>(P) * E * 4);
    outs[nout++] = range_of(rt->recv_rows, static_cast<int64_t>(P) * 8);
    outs[nout++] = range_of(rt->scratch, sbytes);
    if (!disjoint(ins, nin, outs, nout))
        return ATOM_ERR_INVALID_ARG;
    MoeRouteArgs& a = p->a;
    a = MoeRouteArgs{};
    for (int r = 0; r < P; ++r) {
        a.ids[r] = n > 0 ? rt->expert_ids[r] : nullptr;
        a.pos[r] = n > 0 ? rt->positions[r] : nullptr;
    }
    a.counts = rt->counts;
    a.recv = rt->recv_rows;
    a.n = n;
    a.nch = moe_chunks(n);
    // Each placing workgroup rebuilds the per-expert offsets (E x P counts)
    // once, so the placing grid is bounded (~1024) and strides over chunks.
    a.groups = std::max(1, std::min(a.nch, 1024 / P));
    a.P = P;
    a.E = E;
    a.per = E / P;
    a.partial = static_cast<int32_t*>(rt->scratch);
    p->scan_threads = static_cast<int32_t>(ceil_div(E, 64) * 64);
    // Small routings (up to kMoeSmallEntries entries per rank) run as one
    // workgroup of one wave per rank when its counters fit in LDS.
    p->small = n <= kMoeSmallEntries &&
               (static_cast<int64_t>(P) * E + E + 64 * P) * 4 <= kMoeSmallLds;
    return ATOM_OK;
}

atom_status plan_moe_move(const atom_moe_routing* rt, bool combine, const void* const* src,
                          const float* const* w, void* const* dst, int64_t cap, int64_t row_elems,
                          atom_dtype dtype, const atom_config* cfg, MoeMovePlan* p)
{
    if (!p)
        return ATOM_ERR_INVALID_ARG;
    if (atom_status st = check_routing(rt); st != ATOM_OK)
        return st;
    Cfg c;
    if (atom_status st = read_cfg(cfg, &c); st != ATOM_OK)
        return st;
    if (c.flags & (ATOM_F_STAGED | ATOM_F_XCD_ORDER))
        return ATOM_ERR_UNSUPPORTED;
    const int es = esize_of(dtype);
    const int P = rt->nranks;
    const int64_t T = rt->tokens, k = rt->topk;
    int64_t row_bytes = 0, tok_bytes = 0, cap_bytes = 0;
    if (es == 0 || row_elems < 1 || cap < 0 || cap > INT32_MAX || !mul_ok(row_elems, es, &row_bytes) ||
        !mul_ok(T, row_bytes, &tok_bytes) || !mul_ok(cap, row_bytes, &cap_bytes))
        return ATOM_ERR_INVALID_ARG;
    if (T > 0 && (!src || !dst || (combine && !w)))
        return ATOM_ERR_INVALID_ARG;
    // dispatch reads T rows per rank and writes cap rows per rank; combine
    // reads cap rows per rank (and T*k weights) and writes T rows per rank.
    const int64_t src_bytes = combine ? cap_bytes : tok_bytes;
    const int64_t dst_bytes = combine ? tok_bytes : cap_bytes;
    bool vec = row_bytes % kVecBytes == 0;
    Range ins[2 * kMaxRanks + 2 * kMaxRanks], outs[kMaxRanks];
    int nin = 0, nout = 0;
    for (int r = 0; r < P && T > 0; ++r) {
        if (!buffer_ok(src[r], src_bytes, es) || !buffer_ok(dst[r], dst_bytes, es))
            return ATOM_ERR_INVALID_ARG;
        if (combine && !buffer_ok(w[r], T * k * 4, 4))
            return ATOM_ERR_INVALID_ARG;
        vec = vec && aligned(src[r], kVecBytes) && aligned(dst[r], kVecBytes);
        ins[nin++] = range_of(src[r], src_bytes);
        if (combine)
            ins[nin++] = range_of(w[r], T * k * 4);
        ins[nin++] = range_of(rt->expert_ids[r], T * k * 4);
        ins[nin++] = range_of(rt->positions[r], T * k * 4);
        outs[nout++] = range_of(dst[r], dst_bytes);
    }
    if (!disjoint(ins, nin, outs, nout))
        return ATOM_ERR_INVALID_ARG;
    MoeMoveArgs& a = p->a;
    a = MoeMoveArgs{};
    for (int r = 0; r < P && T > 0; ++r) {
        a.src[r] = static_cast<const char*>(src[r]);
        a.dst[r] = static_cast<char*>(dst[r]);
        a.ids[r] = rt->expert_ids[r];
        a.pos[r] = rt->positions[r];
        a.w[r] = combine ? w[r] : nullptr;
    }
    // Tiles: one piece of one token row, lanes * U 16-byte slots. 64-lane
    // tiles keep many waves in flight per CU, as for the zero-staging fan-out
    // and reduce. Measured on MI355X (8 x 512 tokens x 7168 bf16, top-8):
    // dispatch is fastest with 8 slots per lane (8 KiB pieces; 256 x 4 was
    // 4 % slower), combine with 2 (each slot has k loads in flight; 256 x 1
    // was 9 % slower).
    p->wg = c.lanes ? c.lanes : 64;
    p->U = c.stages ? c.stages : (combine ? 2 : 8);
    a.T = T;
    a.cap = cap;
    a.row_bytes = row_bytes;
    a.piece_bytes = static_cast<int64_t>(p->wg) * p->U * kVecBytes;
    // A buffer or a row size off 16-byte alignment: one tile per token row,
    // its lanes striding over the row's elements (the same arithmetic, in
    // the same order, as the vector path).
    a.elem = vec ? 0 : 1;
    if (!vec) {
        p->wg = c.lanes ? c.lanes : 256;
        p->U = 1;
        a.piece_bytes = row_bytes;
    }
    a.pieces = row_bytes > 0 ? ceil_div(row_bytes, a.piece_bytes) : 0;
    const int64_t ntok = static_cast<int64_t>(P) * T;
    if (a.pieces > 0 && ntok > INT64_MAX / a.pieces)
        return ATOM_ERR_INVALID_ARG;
    a.ntiles = ntok * a.pieces;
    a.P = P;
    a.E = rt->num_experts;
    a.per = rt->num_experts / P;
    a.k = static_cast<int32_t>(k);
    a.dtype = dtype == ATOM_DT_BF16 ? DT_BF16 : DT_F32;
    a.nt_store = (c.flags & ATOM_F_NO_NT) ? 0 : 1;
    p->grid = a.ntiles > 0 ? pick_grid(a.ntiles, c.num_wgs) : 0;
    // Algorithmic bytes: every token row read once and written once per
    // choice (dispatch), or every choice's row read once and the token row
    // written once (combine); plus the ids, positions (and weights) read.
    p->credited_bytes = ntok * ((k + 1) * row_bytes + k * (combine ? 12 : 8));
    return ATOM_OK;
}

void plan_fill_info(const Plan& p, atom_plan_info* info)
{
    std::memset(info, 0, sizeof *info);
    info->kind = p.kind;
    info->nranks = p.P;
    info->staged = (p.exec == EX_SNAC_COPY || p.exec == EX_SNAC_REDUCE) ? 1 : 0;
    info->vector_path = p.vec;
    info->elems_per_rank_in = p.in_elems;
    for (int r = 0; r < kMaxRanks; ++r)
        info->elems_per_rank_out[r] = p.out_elems[r];
    info->credited_bytes = p.credited_bytes;
    info->chunk_bytes = p.chunk_bytes;
    info->num_chunks = info->staged ? p.sa.nchunks : 0;
    info->ring_slots = p.slots;
    const int64_t rows = (p.exec == EX_REDUCE && p.ra.grid_parts > 0)  ? p.ra.grid_parts
                         : (p.exec == EX_COPY && p.ca.grid_segs > 0) ? p.ca.grid_segs
                                                                       : 1;
    info->num_wgs = p.exec == EX_NONE ? 0 : static_cast<int32_t>(p.grid * rows);
    if (p.exec == EX_NONE)
        return;
    info->lanes = p.wg;
    info->stages = p.U;
    info->grid_rows = static_cast<int32_t>(rows);
    info->shifted = (p.exec == EX_REDUCE && p.ra.shifted) || (p.exec == EX_COPY && p.ca.shifted) ||
                            ((p.exec == EX_SNAC_COPY || p.exec == EX_SNAC_REDUCE) && p.snac_shifted)
                        ? 1
                        : 0;
    const bool staged = p.exec == EX_SNAC_COPY || p.exec == EX_SNAC_REDUCE;
    info->snac_lead = staged ? p.sa.lead : 0;
    info->snac_tasks = staged ? p.sa.ntasks : 0;
    info->snac_tagged = staged ? p.sa.tagged : 0;
    switch (p.exec) {
    case EX_REDUCE: info->streaming_stores = p.ra.nt_store; break;
    case EX_COPY: info->streaming_stores = p.ca.nt_store; break;
    default: info->streaming_stores = p.sa.nt_store; break;
    }
}

// Table 3: R*tau rounded to the closest power of two (ties upward).
int64_t bdp_chunk_bytes(double bytes_per_s, double round_trip_s)
{
    const double x = bytes_per_s * round_trip_s;
    if (!(x >= 1.0) || !std::isfinite(x))
        return 0;
    if (x >= 4.0e18)
        return int64_t(1) << 62;
    int e;
    std::frexp(x, &e);           // x = m * 2^e, m in [0.5, 1): 2^(e-1) <= x < 2^e
    const double lo = std::ldexp(1.0, e - 1), hi = std::ldexp(1.0, e);
    return static_cast<int64_t>((x - lo < hi - x) ? lo : hi);
}

}  // namespace atom
