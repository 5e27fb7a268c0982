// k_moe.hip -- expert-parallel MoE dispatch and combine on gfx950.
//
// "Purlin: Separating Orchestration from the Datapath of Collectives"
// (arXiv 2609.36954), Table 2: expert parallelism dispatches tokens to
// experts and combines the expert outputs, with AllToAll(V) as the
// collective. Dispatch here is the AllToAllV whose destinations are the
// experts (rows of expert e from every source in rank order, each source's
// rows in entry order; a rank's buffer holds its experts back to back);
// combine is the way back, a weighted sum over each token's k choices.
//
// Routing (metadata only): one workgroup for up to 256 entries per rank
// (k_moe_route_small, the decode case), else three launches:
//   k_moe_rank   one wave per chunk of 256 entries of one rank: the rank of
//                every entry among the chunk's entries with the same expert,
//                in entry order (in each 64-entry step the lanes holding one
//                expert are matched by ballots over the id's bits; an LDS
//                counter per expert carries over between steps), and the
//                chunk's histogram;
//   k_moe_prefix one workgroup per rank, one thread per expert: rows of
//                expert e in the rank's earlier chunks, and the rank's
//                total for e (the counts);
//   k_moe_place  one workgroup per rank and group of chunks (at most ~1024
//                in all): from the counts, the rows of each expert from
//                earlier ranks and (a prefix sum over the experts) the rows
//                of the earlier experts of the same rank, built once per
//                workgroup; position = those + chunk prefix + rank in chunk.
// Movement (HBM bound; a tile is one piece of a token row, 64 lanes by
// default, so that many small workgroups keep each CU's memory queue full):
//   k_moe_dispatch  the token row is loaded once (16-byte vectors) and
//                   stored once per valid choice (non-temporal);
//   k_moe_combine   the k rows of a token are loaded together, then
//                   accumulated in binary32 by fused multiply-adds in choice
//                   order from +0 and rounded once.
#include "atom_dev.hpp"
#include "launch.hpp"

namespace atom {

namespace {

// Ranks one 64-entry step of entries [i0 + s*64, ...) of one rank against the
// per-expert counters `cnt` (LDS, this wave's own): returns, for a valid
// entry, the number of earlier entries with its expert (earlier steps
// included), and -1 for an invalid one. The callers store a batch of steps'
// ranks together, so no store's completion is waited for between steps. The lanes holding the same expert
// are found with one ballot per bit of the expert id (a lane keeps the
// lanes that agree with it on every bit), so an entry's rank within the
// step is the number of such lanes below it, and the highest of them adds
// the group's size to the expert's counter.
__device__ __forceinline__ int32_t rank_step(const MoeRouteArgs& a, int64_t i, int64_t i1, int e,
                                             int32_t* cnt)
{
    const bool valid = i < i1 && e >= 0 && e < a.E;
    unsigned long long same = __ballot(valid);
    const int nbits = a.E > 1 ? 32 - __clz(a.E - 1) : 0;     // wave-uniform
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const unsigned long long ones = __ballot(valid && bit);
        same &= bit ? ones : ~ones;
    }
    const int below = __builtin_amdgcn_mbcnt_hi(static_cast<unsigned int>(same >> 32),
                                                __builtin_amdgcn_mbcnt_lo(static_cast<unsigned int>(same), 0u));
    const int lane = threadIdx.x & 63;
    int32_t before = 0;
    if (valid)
        before = cnt[e];
    // Every lane has read its counter before any lane writes one: the wave's
    // LDS operations complete in program order.
    if (valid && lane == 63 - __clzll(same))
        cnt[e] = before + __popcll(same);
    return valid ? before + below : -1;
}

__global__ __launch_bounds__(64) void k_moe_rank(const MoeRouteArgs a)
{
    extern __shared__ int32_t cnt[];                  // [E]: rows so far in this chunk
    constexpr int kSteps = kMoeChunk / 64;
    const int r = blockIdx.x / a.nch;
    const int ch = blockIdx.x - r * a.nch;
    const int lane = threadIdx.x;
    for (int e = lane; e < a.E; e += 64)
        cnt[e] = 0;
    const int64_t i0 = static_cast<int64_t>(ch) * kMoeChunk;
    const int64_t i1 = i0 + kMoeChunk < a.n ? i0 + kMoeChunk : a.n;
    // The chunk's ids, all loads in flight at once.
    int ids[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int64_t i = i0 + s * 64 + lane;
        ids[s] = i < i1 ? a.ids[r][i] : -1;
    }
    __syncthreads();
    int32_t rk[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
        rk[s] = rank_step(a, i0 + s * 64 + lane, i1, ids[s], cnt);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int64_t i = i0 + s * 64 + lane;
        if (i < i1)
            a.pos[r][i] = rk[s];
    }
    __syncthreads();
    int32_t* part = a.partial + (static_cast<int64_t>(r) * a.nch + ch) * a.E;
    for (int e = lane; e < a.E; e += 64)
        part[e] = cnt[e];
}

// The whole routing in one workgroup for decode-sized batches: wave r
// ranks rank r's entries, 64 at a time in entry order, into its own LDS
// counters (so each entry's rank counts every earlier entry of the rank,
// with no chunk partials); then the block writes the counts, scans the
// expert totals and places every entry (earlier experts of the rank +
// earlier ranks + rank among the rank's entries). One launch instead of
// three.
__global__ __launch_bounds__(1024) void k_moe_route_small(const MoeRouteArgs a)
{
    extern __shared__ int32_t lds[];                  // [P][E] counts, [E] prefix, [nthr] partials
    const int nthr = blockDim.x;                      // 64 * P
    const int tid = threadIdx.x;
    // This wave's rank, made provably wave-uniform so that its pointers are
    // read once into scalar registers (a per-lane index would fetch the
    // pointer from the argument block before every access).
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int32_t* const ids_w = a.ids[w];
    int32_t* const pos_w = a.pos[w];
    int32_t* cnt = lds;
    int32_t* incl = lds + a.P * a.E;
    int32_t* part = incl + a.E;
    for (int q = tid; q < a.P * a.E; q += nthr)
        cnt[q] = 0;
    const int lane = tid & 63;
    const int64_t nsteps = (a.n + 63) / 64;           // the same for every wave
    constexpr int kB = 16;                            // steps whose loads are in flight together
    __syncthreads();
    for (int64_t s0 = 0; s0 < nsteps; s0 += kB) {
        int ev[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int64_t i = (s0 + u) * 64 + lane;
            ev[u] = i < a.n ? ids_w[i] : -1;
        }
        int32_t rk[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u)
            rk[u] = s0 + u < nsteps ? rank_step(a, (s0 + u) * 64 + lane, a.n, ev[u], cnt + w * a.E) : -1;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int64_t i = (s0 + u) * 64 + lane;
            if (i < a.n)
                pos_w[i] = rk[u];
        }
    }
    __syncthreads();
    // counts, and the totals of each expert over the ranks
    for (int e = tid; e < a.E; e += nthr) {
        int32_t tot = 0;
        for (int r = 0; r < a.P; ++r) {
            a.counts[static_cast<int64_t>(r) * a.E + e] = cnt[r * a.E + e];
            tot += cnt[r * a.E + e];
        }
        incl[e] = tot;
    }
    __syncthreads();
    // inclusive prefix of the totals over the experts
    const int m = (a.E + nthr - 1) / nthr;
    int32_t run = 0;
    for (int u = 0; u < m; ++u) {
        const int e = tid * m + u;
        if (e < a.E) {
            run += incl[e];
            incl[e] = run;
        }
    }
    part[tid] = run;
    __syncthreads();
    for (int d = 1; d < nthr; d <<= 1) {
        const int32_t v = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    const int32_t off = tid > 0 ? part[tid - 1] : 0;
    for (int u = 0; u < m; ++u) {
        const int e = tid * m + u;
        if (e < a.E)
            incl[e] += off;
    }
    __syncthreads();
    // Each lane reads back the ranks it wrote itself in the ranking loop,
    // kB steps of loads at a time.
    for (int64_t s0 = 0; s0 < nsteps; s0 += kB) {
        int32_t pv[kB];
        int ev[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int64_t i = (s0 + u) * 64 + lane;
            pv[u] = i < a.n ? pos_w[i] : -1;
            ev[u] = i < a.n ? ids_w[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int64_t i = (s0 + u) * 64 + lane;
            if (i < a.n && pv[u] >= 0) {
                const int e = ev[u];
                const int first = (e / a.per) * a.per;
                int32_t cross = 0;
                for (int r = 0; r < w; ++r)
                    cross += cnt[r * a.E + e];
                const int32_t base = (e > 0 ? incl[e - 1] : 0) - (first > 0 ? incl[first - 1] : 0);
                pos_w[i] = pv[u] + base + cross;
            }
        }
    }
    for (int j = tid; j < a.P; j += nthr)
        a.recv[j] = static_cast<int64_t>(incl[(j + 1) * a.per - 1] - (j > 0 ? incl[j * a.per - 1] : 0));
}

__global__ __launch_bounds__(1024) void k_moe_prefix(const MoeRouteArgs a)
{
    constexpr int kBatch = 16;                        // histogram loads in flight per thread
    const int r = blockIdx.x;
    const int e = threadIdx.x;
    if (e >= a.E)
        return;                                       // (no barrier in this kernel)
    // Walk rank r's chunk histograms of expert e in order, replacing each by
    // the rows of e in the rank's earlier chunks; loads go kBatch at a time.
    int32_t* col = a.partial + static_cast<int64_t>(r) * a.nch * a.E + e;
    int32_t run = 0;
    for (int c0 = 0; c0 < a.nch; c0 += kBatch) {
        int32_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            v[u] = c0 + u < a.nch ? col[static_cast<int64_t>(c0 + u) * a.E] : 0;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (c0 + u < a.nch) {
                col[static_cast<int64_t>(c0 + u) * a.E] = run;
                run += v[u];
            }
        }
    }
    a.counts[static_cast<int64_t>(r) * a.E + e] = run;
}

__global__ __launch_bounds__(256) void k_moe_place(const MoeRouteArgs a)
{
    // LDS: [E] rows of each expert from earlier ranks, [E] inclusive prefix
    // over the experts of each expert's total rows, [256] thread partials.
    extern __shared__ int32_t lds[];
    int32_t* cross = lds;
    int32_t* incl = lds + a.E;
    int32_t* part = lds + 2 * a.E;
    const int r = blockIdx.x / a.groups;              // rank; chunks g, g + groups, ...
    const int g = blockIdx.x - r * a.groups;
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;                      // 256
    for (int e = tid; e < a.E; e += nthr) {
        int32_t before = 0, tot = 0;
        for (int q = 0; q < a.P; ++q) {
            const int32_t c = a.counts[static_cast<int64_t>(q) * a.E + e];
            before += q < r ? c : 0;
            tot += c;
        }
        cross[e] = before;
        incl[e] = tot;
    }
    __syncthreads();
    // Inclusive prefix of the totals over the experts: each thread scans m
    // consecutive experts, the thread sums are scanned in LDS, then added.
    const int m = (a.E + nthr - 1) / nthr;
    int32_t run = 0;
    for (int u = 0; u < m; ++u) {
        const int e = tid * m + u;
        if (e < a.E) {
            run += incl[e];
            incl[e] = run;
        }
    }
    part[tid] = run;
    __syncthreads();
    for (int d = 1; d < nthr; d <<= 1) {
        const int32_t v = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    const int32_t off = tid > 0 ? part[tid - 1] : 0;
    for (int u = 0; u < m; ++u) {
        const int e = tid * m + u;
        if (e < a.E)
            incl[e] += off;
    }
    __syncthreads();
    // position = earlier experts of the rank + earlier ranks + earlier
    // chunks of this rank + rank within the chunk
    for (int ch = g; ch < a.nch; ch += a.groups) {
        const int32_t* chunk_before = a.partial + (static_cast<int64_t>(r) * a.nch + ch) * a.E;
        const int64_t i0 = static_cast<int64_t>(ch) * kMoeChunk;
        const int64_t i1 = i0 + kMoeChunk < a.n ? i0 + kMoeChunk : a.n;
        for (int64_t i = i0 + tid; i < i1; i += nthr) {
            const int32_t p = a.pos[r][i];
            if (p >= 0) {
                const int e = a.ids[r][i];
                const int first = (e / a.per) * a.per;
                const int32_t base = (e > 0 ? incl[e - 1] : 0) - (first > 0 ? incl[first - 1] : 0);
                a.pos[r][i] = p + base + cross[e] + chunk_before[e];
            }
        }
    }
    if (blockIdx.x == 0)
        for (int j = tid; j < a.P; j += nthr)
            a.recv[j] = static_cast<int64_t>(incl[(j + 1) * a.per - 1] - (j > 0 ? incl[j * a.per - 1] : 0));
}

// Token (r, t) of tile `tile`.
__device__ __forceinline__ void token_of(const MoeMoveArgs& a, int64_t tile, int* r, int64_t* t)
{
    *r = static_cast<int>(tile / a.T);
    *t = tile - static_cast<int64_t>(*r) * a.T;
}

// The k choices of token (r, t), read once: lane c of every wave loads
// choice c, then readlane makes each choice's expert-side row address (or
// nullptr for a dropped entry) and weight wave-uniform, so the row loops
// below issue their 16-byte accesses with no metadata load in between.
// KMAX >= k bounds the registers the choices take.
template <int KMAX>
struct Choices {
    char* row[KMAX];
    float w[KMAX];
    uint32_t live;                    // bit c: choice c lands (valid id, position < cap)
};

template <int KMAX>
__device__ __forceinline__ Choices<KMAX> token_choices(const MoeMoveArgs& a, int r, int64_t t,
                                                       char* const* side, bool weights)
{
    const int wl = threadIdx.x & 63;
    int my_e = -1, my_p = -1;
    float my_w = 0.0f;
    if (wl < a.k) {
        my_e = a.ids[r][t * a.k + wl];
        my_p = a.pos[r][t * a.k + wl];
        if (weights)
            my_w = a.w[r][t * a.k + wl];
    }
    Choices<KMAX> ch;
    ch.live = 0;
#pragma unroll
    for (int c = 0; c < KMAX; ++c) {
        const int e = __builtin_amdgcn_readlane(my_e, c);
        const int p = __builtin_amdgcn_readlane(my_p, c);
        ch.w[c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), c));
        const bool ok = c < a.k && e >= 0 && e < a.E && p >= 0 && p < a.cap;
        ch.row[c] = ok ? side[e / a.per] + static_cast<int64_t>(p) * a.row_bytes : nullptr;
        ch.live |= ok ? (1u << c) : 0u;
    }
    return ch;
}

// A tile is one piece of one token row: piece_bytes = blockDim.x * U * 16
// bytes starting at piece * piece_bytes (the row's last piece may be short).
__device__ __forceinline__ int64_t piece_of(const MoeMoveArgs& a, int64_t tile, int* r, int64_t* t)
{
    const int64_t tok = tile / a.pieces;
    token_of(a, tok, r, t);
    return (tile - tok * a.pieces) * a.piece_bytes;
}

template <int KMAX, int U>
__global__ __launch_bounds__(256) void k_moe_dispatch(const MoeMoveArgs a)
{
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const bool nt = a.nt_store != 0;
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        int r;
        int64_t t;
        const int64_t b0 = piece_of(a, tile, &r, &t);
        // The token's own row does not depend on the routing: its loads are
        // issued before the choices are read, so the two latencies overlap.
        const char* src = a.src[r] + t * a.row_bytes;
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t o = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
            if (o < a.row_bytes)
                x[u] = ld16_stream(src + o);
        }
        const Choices<KMAX> ch = token_choices<KMAX>(a, r, t, a.dst, false);
#pragma unroll
        for (int c = 0; c < KMAX; ++c) {
            if ((ch.live >> c) & 1u) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t off = static_cast<uint32_t>(u * nthr + lane) * kVecBytes;
                    if (b0 + off < a.row_bytes)
                        st16(ch.row[c] + b0, off, x[u], nt);
                }
            }
        }
    }
}

// Element-wise dispatch (a buffer or the row size off 16-byte alignment):
// one tile per token row, each lane copying elements of E bytes (the
// element size) with a stride of the workgroup.
template <typename E, int KMAX>
__global__ __launch_bounds__(256) void k_moe_dispatch_elem(const MoeMoveArgs a)
{
    const int64_t n = a.row_bytes / static_cast<int64_t>(sizeof(E));
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        int r;
        int64_t t;
        token_of(a, tile, &r, &t);
        const Choices<KMAX> ch = token_choices<KMAX>(a, r, t, a.dst, false);
        const E* src = reinterpret_cast<const E*>(a.src[r] + t * a.row_bytes);
        for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
            const E v = src[i];
#pragma unroll
            for (int c = 0; c < KMAX; ++c)
                if ((ch.live >> c) & 1u)
                    reinterpret_cast<E*>(ch.row[c])[i] = v;
        }
    }
}

// Accumulators of one 16-byte slot: 8 bf16 or 4 fp32 elements.
template <typename T> struct FmaAcc;

template <> struct FmaAcc<uint16_t> {
    float v[8];
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = 0.0f;
    }
    __device__ __forceinline__ void fma(float w, u32x4 x)
    {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[2 * q] = __builtin_fmaf(w, bf16_lo(x[q]), v[2 * q]);
            v[2 * q + 1] = __builtin_fmaf(w, bf16_hi(x[q]), v[2 * q + 1]);
        }
    }
    __device__ __forceinline__ u32x4 pack() const
    {
        u32x4 r;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            r[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
        return r;
    }
};

template <> struct FmaAcc<float> {
    float v[4];
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[q] = 0.0f;
    }
    __device__ __forceinline__ void fma(float w, u32x4 x)
    {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[q] = __builtin_fmaf(w, __uint_as_float(x[q]), v[q]);
    }
    __device__ __forceinline__ u32x4 pack() const
    {
        u32x4 r;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            r[q] = __float_as_uint(v[q]);
        return r;
    }
};

template <typename T, int KMAX>
__global__ __launch_bounds__(256) void k_moe_combine(const MoeMoveArgs a)
{
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const bool nt = a.nt_store != 0;
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        int r;
        int64_t t;
        const int64_t p0 = piece_of(a, tile, &r, &t);
        const int64_t p1 = p0 + a.piece_bytes < a.row_bytes ? p0 + a.piece_bytes : a.row_bytes;
        const Choices<KMAX> ch = token_choices<KMAX>(a, r, t, const_cast<char* const*>(a.src), true);
        char* dst = a.dst[r] + t * a.row_bytes;
        for (int64_t b0 = p0; b0 < p1; b0 += static_cast<int64_t>(nthr) * kVecBytes) {
            const int64_t o = b0 + static_cast<int64_t>(lane) * kVecBytes;
            const bool in_row = o < a.row_bytes;
            // All of the token's rows for this slot in flight at once.
            u32x4 y[KMAX];
#pragma unroll
            for (int c = 0; c < KMAX; ++c)
                if (((ch.live >> c) & 1u) && in_row)
                    y[c] = ld16_stream(ch.row[c] + o);
            FmaAcc<T> acc;
            acc.zero();
#pragma unroll
            for (int c = 0; c < KMAX; ++c)
                if ((ch.live >> c) & 1u)
                    acc.fma(ch.w[c], y[c]);
            if (in_row)
                st16(dst + b0, static_cast<uint32_t>(lane) * kVecBytes, acc.pack(), nt);
        }
    }
}

// Element-wise combine: one tile per token row; each element is the same
// chain of binary32 fused multiply-adds in choice order from +0 as in the
// vector path, rounded once.
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void k_moe_combine_elem(const MoeMoveArgs a)
{
    const int64_t n = a.row_bytes / static_cast<int64_t>(sizeof(T));
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        int r;
        int64_t t;
        token_of(a, tile, &r, &t);
        const Choices<KMAX> ch = token_choices<KMAX>(a, r, t, const_cast<char* const*>(a.src), true);
        char* dst = a.dst[r] + t * a.row_bytes;
        for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < KMAX; ++c)
                if ((ch.live >> c) & 1u)
                    acc = __builtin_fmaf(ch.w[c], Elem<T>::load(ch.row[c], i), acc);
            Elem<T>::store(dst, i, acc);
        }
    }
}

}  // namespace

hipError_t launch_moe_route(const MoeRoutePlan& p, hipStream_t stream)
{
    const MoeRouteArgs& a = p.a;
    if (a.P < 1 || a.P > kMaxRanks || a.E < 1 || a.E > 1024 || a.nch < 1 || a.per < 1 ||
        a.groups < 1 || a.groups > a.nch || p.scan_threads < a.E || p.scan_threads > 1024 ||
        p.scan_threads % 64 != 0)
        return hipErrorInvalidValue;
    if (p.small) {
        const size_t lds = static_cast<size_t>(a.P * a.E + a.E + 64 * a.P) * sizeof(int32_t);
        if (a.n > kMoeSmallEntries || lds > kMoeSmallLds)
            return hipErrorInvalidValue;
        k_moe_route_small<<<dim3(1), dim3(64 * a.P), lds, stream>>>(a);
        return hipGetLastError();
    }
    const unsigned nb = static_cast<unsigned>(a.P) * static_cast<unsigned>(a.nch);
    k_moe_rank<<<dim3(nb), dim3(64), static_cast<size_t>(a.E) * sizeof(int32_t), stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    k_moe_prefix<<<dim3(a.P), dim3(p.scan_threads), 0, stream>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const unsigned np = static_cast<unsigned>(a.P) * static_cast<unsigned>(a.groups);
    k_moe_place<<<dim3(np), dim3(256), static_cast<size_t>(2 * a.E + 256) * sizeof(int32_t), stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_moe_move(const MoeMovePlan& p, bool combine, hipStream_t stream)
{
    const MoeMoveArgs& a = p.a;
    if (a.ntiles == 0)
        return hipSuccess;
    const dim3 grid(static_cast<unsigned>(p.grid)), block(static_cast<unsigned>(p.wg));
    const int kmax = a.k <= 2 ? 2 : a.k <= 4 ? 4 : a.k <= 8 ? 8 : 16;
    if (a.elem) {
        const int es = a.dtype == DT_BF16 ? 2 : 4;
        if (p.grid < 1 || a.k < 1 || a.k > kMoeMaxTopk || a.per < 1 || a.row_bytes % es != 0 ||
            p.wg < 64 || p.wg > 256 || p.wg % 64 != 0 || a.pieces != 1 || a.piece_bytes != a.row_bytes)
            return hipErrorInvalidValue;
        const bool bf = a.dtype == DT_BF16;
#define ATOM_MOE_ELEM(KM)                                                                     \
    case KM:                                                                                  \
        if (combine)                                                                          \
            bf ? k_moe_combine_elem<uint16_t, KM><<<grid, block, 0, stream>>>(a)              \
               : k_moe_combine_elem<float, KM><<<grid, block, 0, stream>>>(a);                \
        else                                                                                  \
            bf ? k_moe_dispatch_elem<uint16_t, KM><<<grid, block, 0, stream>>>(a)             \
               : k_moe_dispatch_elem<uint32_t, KM><<<grid, block, 0, stream>>>(a);            \
        break;
        switch (kmax) {
        ATOM_MOE_ELEM(2) ATOM_MOE_ELEM(4) ATOM_MOE_ELEM(8) ATOM_MOE_ELEM(16)
        }
#undef ATOM_MOE_ELEM
        return hipGetLastError();
    }
    if (p.grid < 1 || a.k < 1 || a.k > kMoeMaxTopk || a.per < 1 || a.row_bytes % kVecBytes != 0 ||
        p.wg < 64 || p.wg > 256 || p.wg % 64 != 0 ||
        a.piece_bytes != static_cast<int64_t>(p.wg) * p.U * kVecBytes || a.pieces < 1 ||
        a.pieces * a.piece_bytes < a.row_bytes)
        return hipErrorInvalidValue;
    if (combine) {
        const bool bf = a.dtype == DT_BF16;
        switch (kmax) {
#define ATOM_MOE_COMBINE(KM)                                                         \
    case KM:                                                                         \
        if (bf)                                                                      \
            k_moe_combine<uint16_t, KM><<<grid, block, 0, stream>>>(a);             \
        else                                                                         \
            k_moe_combine<float, KM><<<grid, block, 0, stream>>>(a);                \
        break;
        ATOM_MOE_COMBINE(2) ATOM_MOE_COMBINE(4) ATOM_MOE_COMBINE(8) ATOM_MOE_COMBINE(16)
#undef ATOM_MOE_COMBINE
        }
    } else {
#define ATOM_MOE_DISPATCH(UU)                                                        \
    case UU:                                                                         \
        switch (kmax) {                                                              \
        case 2: k_moe_dispatch<2, UU><<<grid, block, 0, stream>>>(a); break;         \
        case 4: k_moe_dispatch<4, UU><<<grid, block, 0, stream>>>(a); break;         \
        case 8: k_moe_dispatch<8, UU><<<grid, block, 0, stream>>>(a); break;         \
        default: k_moe_dispatch<16, UU><<<grid, block, 0, stream>>>(a); break;       \
        }                                                                            \
        break;
        switch (p.U) {
        ATOM_MOE_DISPATCH(1) ATOM_MOE_DISPATCH(2) ATOM_MOE_DISPATCH(4) ATOM_MOE_DISPATCH(8)
        default: return hipErrorInvalidValue;
        }
#undef ATOM_MOE_DISPATCH
    }
    return hipGetLastError();
}

}  // namespace atom
