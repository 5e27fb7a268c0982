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
// Routing (three small launches, metadata only):
//   k_moe_rank   one wave per chunk of 1024 entries of one rank: the rank of
//                every entry among the chunk's entries with the same expert,
//                in entry order (wave ballots group equal ids; an LDS counter
//                per expert carries over between 64-entry steps), and the
//                chunk's histogram;
//   k_moe_scan   one workgroup, one thread per expert: rows of expert e
//                before each (rank, chunk) -- earlier ranks, earlier chunks --
//                and, by a prefix sum over the experts of each rank, the
//                rows of the earlier experts of the same rank;
//   k_moe_place  position = expert base + chunk prefix + rank in chunk.
// Movement (HBM bound, one tile per token row):
//   k_moe_dispatch  the token row is loaded once (16-byte vectors) and
//                   stored once per valid choice (non-temporal);
//   k_moe_combine   the k rows of a token are loaded together, then
//                   accumulated in binary32 by fused multiply-adds in choice
//                   order from +0 and rounded once.
#include "atom_dev.hpp"
#include "launch.hpp"

namespace atom {

namespace {

__global__ __launch_bounds__(64) void k_moe_rank(const MoeRouteArgs a)
{
    extern __shared__ int32_t cnt[];                  // [E]: rows so far in this chunk
    const int r = blockIdx.x / a.nch;
    const int ch = blockIdx.x - r * a.nch;
    const int lane = threadIdx.x;
    for (int e = lane; e < a.E; e += 64)
        cnt[e] = 0;
    __syncthreads();
    const int64_t i0 = static_cast<int64_t>(ch) * kMoeChunk;
    const int64_t i1 = i0 + kMoeChunk < a.n ? i0 + kMoeChunk : a.n;
    for (int64_t b = i0; b < i1; b += 64) {
        const int64_t i = b + lane;
        const int e = i < i1 ? a.ids[r][i] : -1;
        const bool valid = i < i1 && e >= 0 && e < a.E;
        // Lanes with the same expert: peel one id per round (the lowest
        // pending lane's) until every valid lane has its group mask.
        uint64_t todo = __ballot(valid);
        uint64_t mine = 0;
        while (todo != 0) {
            const int leader = __builtin_ctzll(todo);
            const int v = __builtin_amdgcn_readlane(e, leader);
            const bool hit = valid && e == v;
            const uint64_t m = __ballot(hit);
            if (hit)
                mine = m;
            todo &= ~m;
        }
        int32_t before = 0;
        if (valid)
            before = cnt[e];
        // Every lane has read its counter before any lane writes one: the
        // wave's LDS operations complete in program order.
        if (valid) {
            const uint64_t lower = lane == 0 ? 0 : (mine & ((~0ull) >> (64 - lane)));
            a.pos[r][i] = before + __popcll(lower);
            if ((mine >> lane) == 1)                  // the group's highest lane
                cnt[e] = before + __popcll(mine);
        } else if (i < i1) {
            a.pos[r][i] = -1;
        }
    }
    __syncthreads();
    int32_t* part = a.partial + (static_cast<int64_t>(r) * a.nch + ch) * a.E;
    for (int e = lane; e < a.E; e += 64)
        part[e] = cnt[e];
}

__global__ __launch_bounds__(1024) void k_moe_scan(const MoeRouteArgs a)
{
    extern __shared__ int32_t incl[];                 // [E]: totals, then inclusive prefix
    const int e = threadIdx.x;
    int32_t tot = 0;
    if (e < a.E) {
        for (int r = 0; r < a.P; ++r) {
            int32_t from_r = 0;
            for (int ch = 0; ch < a.nch; ++ch) {
                int32_t* q = a.partial + (static_cast<int64_t>(r) * a.nch + ch) * a.E + e;
                const int32_t v = *q;
                *q = tot;                             // rows of e before this chunk
                tot += v;
                from_r += v;
            }
            a.counts[static_cast<int64_t>(r) * a.E + e] = from_r;
        }
        incl[e] = tot;
    }
    __syncthreads();
    for (int d = 1; d < a.E; d <<= 1) {               // Hillis-Steele over the experts
        int32_t v = 0;
        if (e < a.E && e >= d)
            v = incl[e - d];
        __syncthreads();
        if (e < a.E && e >= d)
            incl[e] += v;
        __syncthreads();
    }
    if (e < a.E) {
        const int first = (e / a.per) * a.per;        // the rank's first expert
        const int32_t before_rank = first > 0 ? incl[first - 1] : 0;
        a.base[e] = incl[e] - tot - before_rank;
        if (e - first == a.per - 1)
            a.recv[e / a.per] = static_cast<int64_t>(incl[e] - before_rank);
    }
}

__global__ __launch_bounds__(256) void k_moe_place(const MoeRouteArgs a)
{
    const int r = blockIdx.x / a.nch;
    const int ch = blockIdx.x - r * a.nch;
    const int32_t* before = a.partial + (static_cast<int64_t>(r) * a.nch + ch) * a.E;
    const int64_t i0 = static_cast<int64_t>(ch) * kMoeChunk;
    const int64_t i1 = i0 + kMoeChunk < a.n ? i0 + kMoeChunk : a.n;
    for (int64_t i = i0 + threadIdx.x; i < i1; i += blockDim.x) {
        const int32_t p = a.pos[r][i];
        if (p >= 0) {
            const int e = a.ids[r][i];
            a.pos[r][i] = p + a.base[e] + before[e];
        }
    }
}

// Token (r, t) of tile `tile`.
__device__ __forceinline__ void token_of(const MoeMoveArgs& a, int64_t tile, int* r, int64_t* t)
{
    *r = static_cast<int>(tile / a.T);
    *t = tile - static_cast<int64_t>(*r) * a.T;
}

__device__ __forceinline__ bool entry_ok(const MoeMoveArgs& a, int e, int32_t p)
{
    return e >= 0 && e < a.E && p >= 0 && p < a.cap;
}

template <int U>
__global__ __launch_bounds__(256) void k_moe_dispatch(const MoeMoveArgs a)
{
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const bool nt = a.nt_store != 0;
    const int64_t step = static_cast<int64_t>(nthr) * U * kVecBytes;
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        int r;
        int64_t t;
        token_of(a, tile, &r, &t);
        const int32_t* ids = a.ids[r] + t * a.k;
        const int32_t* pos = a.pos[r] + t * a.k;
        const char* src = a.src[r] + t * a.row_bytes;
        for (int64_t b0 = 0; b0 < a.row_bytes; b0 += step) {
            u32x4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t o = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
                if (o < a.row_bytes)
                    x[u] = ld16_stream(src + o);
            }
            for (int c = 0; c < a.k; ++c) {
                const int e = ids[c];
                const int32_t p = pos[c];
                if (!entry_ok(a, e, p))
                    continue;
                char* dst = a.dst[e / a.per] + static_cast<int64_t>(p) * a.row_bytes;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t o = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
                    if (o < a.row_bytes)
                        st16(dst + o, x[u], nt);
                }
            }
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

template <typename T>
__global__ __launch_bounds__(256) void k_moe_combine(const MoeMoveArgs a)
{
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const bool nt = a.nt_store != 0;
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        int r;
        int64_t t;
        token_of(a, tile, &r, &t);
        const int32_t* ids = a.ids[r] + t * a.k;
        const int32_t* pos = a.pos[r] + t * a.k;
        const float* w = a.w[r] + t * a.k;
        char* dst = a.dst[r] + t * a.row_bytes;
        for (int64_t o = static_cast<int64_t>(lane) * kVecBytes; o - lane * kVecBytes < a.row_bytes;
             o += static_cast<int64_t>(nthr) * kVecBytes) {
            const bool in_row = o < a.row_bytes;
            // All of the token's rows for this slot in flight at once.
            u32x4 y[kMoeMaxTopk];
#pragma unroll
            for (int c = 0; c < kMoeMaxTopk; ++c) {
                if (c < a.k) {
                    const int e = ids[c];
                    const int32_t p = pos[c];
                    if (entry_ok(a, e, p) && in_row)
                        y[c] = ld16_stream(a.src[e / a.per] + static_cast<int64_t>(p) * a.row_bytes + o);
                }
            }
            FmaAcc<T> acc;
            acc.zero();
#pragma unroll
            for (int c = 0; c < kMoeMaxTopk; ++c) {
                if (c < a.k && entry_ok(a, ids[c], pos[c]))
                    acc.fma(w[c], y[c]);
            }
            if (in_row)
                st16(dst + o, acc.pack(), nt);
        }
    }
}

}  // namespace

hipError_t launch_moe_route(const MoeRoutePlan& p, hipStream_t stream)
{
    const MoeRouteArgs& a = p.a;
    if (a.P < 1 || a.P > kMaxRanks || a.E < 1 || a.E > 1024 || a.nch < 1 || a.per < 1 ||
        p.scan_threads < a.E || p.scan_threads > 1024 || p.scan_threads % 64 != 0)
        return hipErrorInvalidValue;
    const unsigned nb = static_cast<unsigned>(a.P) * static_cast<unsigned>(a.nch);
    const size_t lds = static_cast<size_t>(a.E) * sizeof(int32_t);
    k_moe_rank<<<dim3(nb), dim3(64), lds, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    k_moe_scan<<<dim3(1), dim3(p.scan_threads), lds, stream>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    k_moe_place<<<dim3(nb), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_moe_move(const MoeMovePlan& p, bool combine, hipStream_t stream)
{
    const MoeMoveArgs& a = p.a;
    if (a.ntiles == 0)
        return hipSuccess;
    if (p.grid < 1 || a.k < 1 || a.k > kMoeMaxTopk || a.per < 1 || a.row_bytes % kVecBytes != 0)
        return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(p.grid)), block(256);
    if (combine) {
        if (a.dtype == DT_BF16)
            k_moe_combine<uint16_t><<<grid, block, 0, stream>>>(a);
        else
            k_moe_combine<float><<<grid, block, 0, stream>>>(a);
    } else {
        if (p.U != 4)
            return hipErrorInvalidValue;
        k_moe_dispatch<4><<<grid, block, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace atom
