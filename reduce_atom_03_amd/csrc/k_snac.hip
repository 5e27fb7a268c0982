// k_snac.hip -- SNAC (Stage, Notify, And Consume) on one gfx950 device.
//
// "Purlin: Separating Orchestration from the Datapath of Collectives"
// (arXiv 2609.36954): the abstract introduces SNAC as the orchestration
// shared by every collective, derived from the layouts; Figure 6 shows ranks
// staging chunks incrementally while consumers gather them; Table 3 sizes a
// chunk as the bandwidth-delay product; Figures 9 and 10 contrast ordinary
// buffers (staged) with peer-accessible ones (zero staging); Figure 16 runs
// the variable-length collectives on ordinary buffers.
//
// On one device the P ranks are P buffers. The planner turns the layouts into
// a list of segments (kargs.hpp: SnacKind), each a contiguous byte range that
// one stage produces and one consume step delivers:
//   AllGather(V)      copy z_k            -> every output, at z_k's place
//   AllToAll(V)       copy x_r's block j  -> output j, after earlier sources
//   ReduceScatter(V)  sum of partition k  -> output k
//   AllReduce         sum of partition k  -> every output, at partition k
// and the hand-off between a producer and its consumers crosses workgroups
// (and XCDs, each with its own L2) through device memory:
//   Stage   a producer workgroup copies (or reduces in rank order) one piece
//           of a chunk into a slot of the staging ring with agent-coherent
//           stores;
//   Notify  once every wave's stores have completed it counts one piece
//           staged in the slot's count word;
//   Consume a consumer workgroup waits until the word counts all pieces of
//           the chunk staged, reads one piece from the slot with
//           agent-coherent loads, writes it to its destination(s) and counts
//           one piece consumed in the same word, which the producer of the
//           chunk D places later waits for before reuse.
// A slot's word holds both counts (staged in the low 32 bits, consumed in
// the high 32 bits) over every chunk the slot holds in the call, so the
// task that brings both to their final values knows that no other task of
// the call will touch the word again.
// The ring is never touched by ordinary (L2-cached) accesses, so no task
// needs an L2 write-back or invalidation.
//
// Tasks are claimed from one atomic ticket in an order where every task
// depends only on tasks with smaller tickets: producers of chunks 0..E-1,
// then for each later chunk q the consumers of chunk q-E followed by the
// producers of chunk q, then the consumers of the last E chunks, where the
// lead E is at most the ring depth D. The producer of chunk q reuses the
// slot of chunk q-D, whose consumers were claimed D-E chunk steps earlier
// (E = D would make it wait for the consumers claimed just before it). A
// claimed ticket belongs to a running workgroup, so the lowest unfinished
// task can always proceed: no deadlock for any grid size or occupancy. A
// workgroup claims its next ticket only when its task is done: claimed while
// the task runs (to hide the atomic's round trip), the next ticket's task
// waits for the current one, and since adjacent tickets depend on each
// other (a chunk's consumers, then the producers that reuse their slots)
// that chained the tasks; measured on MI355X, the staged AllGather of
// 8 x 64 MiB took 2.7 ms instead of 0.98. Every wait is
// bounded; on expiry the error word is set to the call's sequence number,
// the task is dropped, and the call's later waits give up at once, so the
// grid always drains (a later call, with another number, waits normally).
#include <algorithm>
#include <mutex>

#include "atom_dev.hpp"
#include "launch.hpp"

namespace atom {

namespace {

// A slot word counts staged pieces in its low 32 bits and consumed pieces
// in its high 32 bits.
constexpr unsigned long long kConsumedOne = 1ull << 32;
// 16-byte ring vectors per lane in flight on the shifted consume path (two
// arrays of them are live, so few keep the kernel's register budget).
constexpr int kShiftSlots = 2;

struct Task {
    bool produce;
    int64_t chunk;
    int64_t piece;
};

__device__ __forceinline__ Task decode_task(const SnacArgs& a, int64_t t)
{
    const int64_t G = a.pieces, E = a.lead, Q = a.nchunks;
    const int64_t warm = (Q < E ? Q : E) * G;              // producers of chunks 0..E-1
    const int64_t mid = (Q > E ? Q - E : 0) * 2 * G;       // [consume q-E, produce q]
    Task k;
    if (t < warm) {
        k.produce = true;
        k.chunk = t / G;
        k.piece = t - k.chunk * G;
    } else if (t < warm + mid) {
        const int64_t u = t - warm;
        const int64_t q = E + u / (2 * G);
        const int64_t w = u - (q - E) * 2 * G;
        k.produce = w >= G;
        k.chunk = k.produce ? q : q - E;
        k.piece = k.produce ? w - G : w;
    } else {
        const int64_t u = t - warm - mid;
        k.produce = false;
        k.chunk = (Q > E ? Q - E : 0) + u / G;
        k.piece = u - (u / G) * G;
    }
    return k;
}

// Where a segment's bytes come from and go to.
struct SegGeo {
    const char* src;   // copy stages: the segment's first source byte
    int64_t src_off;   // reduce stages: byte offset of the segment in every source
    int64_t dst_off;   // byte offset in the destination(s)
    int64_t bytes;
    int dst;           // destination index, or -1 for every destination
};

__device__ __forceinline__ SegGeo seg_geo(const SnacArgs& a, int s)
{
    SegGeo g;
    g.bytes = static_cast<int64_t>(a.cnt[s]) * a.row_bytes;
    g.src = nullptr;
    g.src_off = 0;
    if (a.kind == SK_EXCHANGE) {
        const int r = s / a.P, j = s - r * a.P;
        int64_t src_rows = 0, dst_rows = 0;
        for (int jj = 0; jj < j; ++jj)       // source r's rows for earlier destinations
            src_rows += a.cnt[r * a.P + jj];
        for (int rr = 0; rr < r; ++rr)       // earlier sources' rows for destination j
            dst_rows += a.cnt[rr * a.P + j];
        g.src = static_cast<const char*>(a.src[r]) + src_rows * a.row_bytes;
        g.dst_off = dst_rows * a.row_bytes;
        g.dst = j;
        return g;
    }
    int64_t rows = 0;                        // rows of the segments before s
    for (int k = 0; k < s; ++k)
        rows += a.cnt[k];
    const int64_t off = rows * a.row_bytes;
    if (a.kind == SK_GATHER) {
        g.src = static_cast<const char*>(a.src[s]);
        g.dst_off = off;
        g.dst = -1;
    } else if (a.kind == SK_SCATTER) {
        g.src_off = off;
        g.dst_off = 0;
        g.dst = s;
    } else {                                 // SK_ALLRED
        g.src_off = off;
        g.dst_off = off;
        g.dst = -1;
    }
    return g;
}

// Segment and chunk-within-segment of chunk q.
__device__ __forceinline__ void chunk_of(const SnacArgs& a, int64_t q, int* s, int64_t* c)
{
    if (a.interleave) {
        *s = static_cast<int>(q % a.nseg);
        *c = q / a.nseg;
        return;
    }
    int lo = 0, hi = a.nseg - 1;           // largest s with chunk_begin[s] <= q
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.chunk_begin[mid] <= q)
            lo = mid;
        else
            hi = mid - 1;
    }
    *s = lo;
    *c = q - a.chunk_begin[lo];
}

// Lane 0 waits until the count in the word (the low 32 bits, or the high 32
// bits when `consumed`) is at least target, bounded in wall-clock time (the
// per-wait bound and the workgroup's whole-kernel budget, both in ticks of
// the constant-rate device clock). The barrier then holds every wave until
// the count was seen, so the waves' ring loads are issued after it. The
// result is made wave-uniform with readfirstlane so every branch on it is
// uniform. Returns false when the wait gave up (a timeout here, or earlier
// in the same call).
__device__ __forceinline__ bool wait_at_least(const SnacArgs& a, const unsigned long long* flag,
                                              bool consumed, unsigned long long target,
                                              long long t_begin, int* s_ok)
{
    // A count of zero is always met (a slot's first use): no flag load, no
    // barrier. `target` is wave-uniform, so this is a uniform branch.
    if (target == 0)
        return true;
    if (threadIdx.x == 0) {
        int ok = 1;
        const int sh = consumed ? 32 : 0;
        const auto count = [&] { return (flag_load_relaxed(flag) >> sh) & 0xFFFFFFFFull; };
        if (count() < target) {
            const long long w0 = wall_clock64();
            unsigned int it = 0;
            while (count() < target) {
                // Back off: waiting workgroups poll one counter line, and a
                // poll that misses costs the producers memory bandwidth.
                if (it < 8)
                    __builtin_amdgcn_s_sleep(2);
                else
                    __builtin_amdgcn_s_sleep(16);
                if ((++it & 15u) == 0) {
                    const long long now = wall_clock64();
                    if (__hip_atomic_load(a.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.seq ||
                        now - w0 > a.wait_ticks || now - t_begin > a.budget_ticks) {
                        __hip_atomic_store(a.error, a.seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        ok = 0;
                        break;
                    }
                }
            }
        }
        *s_ok = ok;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*s_ok) != 0;
}

// Test hook (atom_config.jitter_us): lane 0 holds its workgroup for a
// pseudo-random 0..jitter_ticks device-clock ticks, drawn from the seed, the
// ticket and the point in the task, so that hand-offs are exercised at
// timings other than the natural ones. The caller's barrier follows.
__device__ __forceinline__ void jitter(const SnacArgs& a, int64_t ticket, uint32_t where)
{
    if (a.jitter_ticks > 0 && threadIdx.x == 0) {
        uint32_t h = a.jitter_seed ^ (static_cast<uint32_t>(ticket) * 0x9E3779B9u) ^ (where * 0x85EBCA6Bu);
        h ^= h >> 16;                      // integer finalizer (avalanche)
        h *= 0x7FEB352Du;
        h ^= h >> 15;
        h *= 0x846CA68Bu;
        h ^= h >> 16;
        const long long d = static_cast<long long>(h % static_cast<uint32_t>(a.jitter_ticks + 1));
        const long long t0 = wall_clock64();
        while (wall_clock64() - t0 < d)
            __builtin_amdgcn_s_sleep(4);
    }
}

// ---- stages (vector path: every stream of the segment 16-byte aligned) ---
// Each fills `bytes` bytes of a ring slot from segment byte `off`. A last
// vector that runs past the segment's end is staged whole: its bytes beyond
// the end are never consumed, and its load stays inside the 16-byte block of
// the segment's last byte.

// Copy: from the segment's source (AllGather, AllToAll).
struct StageCopy {
    // One 16-byte vector of the staged data, from segment byte o.
    __device__ static u32x4 stage_vec(const SnacArgs& a, const SegGeo& g, int64_t o)
    {
        return ld16_stream(g.src + o);
    }
    template <int U>
    __device__ static void produce(const SnacArgs& a, const SegGeo& g, int64_t off, char* dst,
                                   int64_t bytes)
    {
        const char* src = g.src + off;
        const auto ring = ring_rsrc(dst, ceil16(bytes));
        const int lane = threadIdx.x;
        const int nthr = blockDim.x;
        const int64_t step = static_cast<int64_t>(nthr) * U * kVecBytes;
        for (int64_t b0 = 0; b0 < bytes; b0 += step) {
            u32x4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t o = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
                if (o < bytes)
                    x[u] = ld16_stream(src + o);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t o = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
                if (o < bytes)
                    st16_agent(ring, o, x[u]);
            }
        }
    }
};

// Reduce: the segment's range summed over the P inputs in rank order,
// rounded once (ReduceScatter, and its half of the composed AllReduce).
template <typename T, int P>
struct StageReduce {
    __device__ static u32x4 stage_vec(const SnacArgs& a, const SegGeo& g, int64_t o)
    {
        u32x4 x[P];
#pragma unroll
        for (int r = 0; r < P; ++r)
            x[r] = ld16_stream(static_cast<const char*>(a.src[r]) + g.src_off + o);
        SlotAcc<T> acc;
        acc.init(x[0]);
#pragma unroll
        for (int r = 1; r < P; ++r)
            acc.add(x[r]);
        return acc.pack();
    }
    template <int U>
    __device__ static void produce(const SnacArgs& a, const SegGeo& g, int64_t off, char* dst,
                                   int64_t bytes)
    {
        const int64_t base = g.src_off + off;
        const auto ring = ring_rsrc(dst, ceil16(bytes));
        const int lane = threadIdx.x;
        const int nthr = blockDim.x;
        const int64_t step = static_cast<int64_t>(nthr) * U * kVecBytes;
        for (int64_t b0 = 0; b0 < bytes; b0 += step) {
            u32x4 x[U][P];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t o = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
                if (o < bytes) {
#pragma unroll
                    for (int r = 0; r < P; ++r)
                        x[u][r] = ld16_stream(static_cast<const char*>(a.src[r]) + base + o);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t o = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
                if (o < bytes) {
                    SlotAcc<T> acc;
                    acc.init(x[u][0]);
#pragma unroll
                    for (int r = 1; r < P; ++r)
                        acc.add(x[u][r]);
                    st16_agent(ring, o, acc.pack());
                }
            }
        }
    }
};

// Consume (vector path): one piece from the slot to its destination(s). A
// last vector that ends past the segment is written in 2-byte units.
// Stores are aligned to the destination's 128-byte lines: the piece's
// destination starts D bytes past a line (D a multiple of 16, taken from the
// first destination; every destination of an AllGather segment sits at the
// same offset when the outputs share their alignment), and when the piece is
// a whole number of 16-byte vectors (and longer than D), vector v of the
// loop takes piece byte (16 v - D) mod bytes, a rotation of the vectors.
// Each wave's 64 stores then fill whole lines (the first D / 16 vectors
// write the piece's last D bytes), instead of every wave straddling one more
// line than it fills; the ring loads take the offset instead, one line in
// eight. Measured on MI355X: the
// staged AllGatherV of 512 MiB in Zipf(0.125) partitions (segments at
// 16-byte offsets) 1.00 -> 0.90 ms, the time of the uniform AllGather.
template <int U>
__device__ __forceinline__ void consume_vec(const SnacArgs& a, const SegGeo& g, const char* src,
                                            int64_t dst_off, int64_t bytes)
{
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const bool nt = a.nt_store != 0;
    const auto ring = ring_rsrc(src, ceil16(bytes));
    const int q0 = g.dst < 0 ? 0 : g.dst;
    const int q1 = g.dst < 0 ? a.P : g.dst + 1;
    const int64_t step = static_cast<int64_t>(nthr) * U * kVecBytes;
    constexpr int64_t kLine = 128;
    int64_t D = bytes % kVecBytes == 0
                    ? static_cast<int64_t>((reinterpret_cast<uintptr_t>(a.dst[q0]) + dst_off) & (kLine - 1))
                    : 0;
    if (D >= bytes)
        D = 0;
    for (int64_t b0 = 0; b0 < bytes; b0 += step) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
            const int64_t o = v - D < 0 ? v - D + bytes : v - D;
            if (v < bytes)
                x[u] = ld16_agent(ring, o);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
            const int64_t o = v - D < 0 ? v - D + bytes : v - D;
            if (v >= bytes) {
                // past the piece: owned by no lane
            } else if (o + kVecBytes <= bytes) {
                for (int q = q0; q < q1; ++q)
                    st16(static_cast<char*>(a.dst[q]) + dst_off, static_cast<uint32_t>(o), x[u], nt);
            } else {
                // the segment's last, partial vector (only when D = 0)
                for (int q = q0; q < q1; ++q) {
                    uint16_t* d = reinterpret_cast<uint16_t*>(static_cast<char*>(a.dst[q]) + dst_off + o);
                    for (int h = 0; h < (bytes - o) / 2; ++h)
                        d[h] = static_cast<uint16_t>(x[u][h >> 1] >> (16 * (h & 1)));
                }
            }
        }
    }
}

// Consume (shifted path): the piece sits in the ring at `src`, at its
// sources' offset from 16-byte alignment, and a destination at another. As
// the zero-staging shifted copy: vector v holds ring bytes [16v, 16v + 16)
// of the address space, from the one holding the piece's first byte to one
// past the one holding its last; each lane loads its vector (agent-coherent,
// never outside the ring: a slot's padding covers both ends), takes vector
// v - 1 from the lane below (lane 0 from the previous row, or a load of its
// own for the wave's first), and writes the destination slot holding the
// tail of v - 1 and the head of v: one 16-byte store, or element-wise stores
// for the slots at the piece's two ends. Each destination's offset d from
// the ring is taken on its own (wave-uniform).
template <int U>
__device__ __forceinline__ void consume_shift(const SnacArgs& a, const SegGeo& g, const char* src,
                                              int64_t dst_off, int64_t bytes, int es)
{
    if (bytes <= 0)
        return;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t nwave = blockDim.x >> 6;
    const bool nt = a.nt_store != 0;
    const int q0 = g.dst < 0 ? 0 : g.dst;
    const int q1 = g.dst < 0 ? a.P : g.dst + 1;
    const int64_t A = static_cast<int64_t>(reinterpret_cast<uintptr_t>(src));
    const int64_t vlo = A >> 4, vhi = (A + bytes - 1) >> 4;
    const auto ring = ring_rsrc(src - (A & 15), (vhi - vlo + 1) * kVecBytes);
    const u32x4 zero = {0, 0, 0, 0};
    // Rows of 64 vectors start where the first destination's slots begin a
    // 128-byte line (the slot of vector v sits at 16 v + (D - A - d)), so
    // each wave's stores fill whole lines; the first row may start before
    // the piece.
    const int64_t m0 = static_cast<int64_t>(reinterpret_cast<uintptr_t>(a.dst[q0]) + dst_off) - A;
    const int64_t vs = vlo - ((vlo + ((m0 - (m0 & 15)) >> 4)) & 7);
    for (int64_t w0 = vs + wave * 64 * U; w0 <= vhi + 1; w0 += nwave * 64 * U) {
        u32x4 R[U], L[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = w0 + u * 64 + lane;
            R[u] = v >= vlo && v <= vhi ? ld16_agent(ring, (v - vlo) * kVecBytes) : zero;
        }
        u32x4 carry = zero;
        if (lane == 0 && w0 - 1 >= vlo && w0 - 1 <= vhi)
            carry = ld16_agent(ring, (w0 - 1 - vlo) * kVecBytes);
#pragma unroll
        for (int u = 0; u < U; ++u)
            L[u] = from_lane_below(R[u], u == 0 ? carry : lane63(R[u - 1]));
        for (int q = q0; q < q1; ++q) {
            char* const D = static_cast<char*>(a.dst[q]) + dst_off;
            const int d = static_cast<int>((reinterpret_cast<uintptr_t>(D) - static_cast<uint64_t>(A)) & 15);
            // slot of vector v: ring bytes [16v - d, 16v - d + 16), stored
            // 16-byte aligned at D + (16v - d - A); wave-uniform base
            char* const wbase = D + ((w0 - vlo) << 4) - (A & 15) - d;   // may precede D (unused)
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
                    store_slot_part(wbase + off, slot, p0, p1, es);
            }
        }
    }
}

// ---- element-wise path: a segment with a stream off 16-byte alignment ----
// Elements of E bytes (the element type's size) move one per lane at a time;
// ring accesses keep the agent-coherent policy.

template <typename E>
__device__ __forceinline__ E ring_load(__amdgpu_buffer_rsrc_t r, int64_t off);
template <>
__device__ __forceinline__ uint16_t ring_load<uint16_t>(__amdgpu_buffer_rsrc_t r, int64_t off)
{
    return static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, kCpolSc1));
}
template <>
__device__ __forceinline__ uint32_t ring_load<uint32_t>(__amdgpu_buffer_rsrc_t r, int64_t off)
{
    return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, kCpolSc1));
}
__device__ __forceinline__ void ring_store(__amdgpu_buffer_rsrc_t r, int64_t off, uint16_t v)
{
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<short>(v), r, static_cast<int>(off), 0, kCpolSc1);
}
__device__ __forceinline__ void ring_store(__amdgpu_buffer_rsrc_t r, int64_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(static_cast<int>(v), r, static_cast<int>(off), 0, kCpolSc1);
}

// Stage element by element: a copy, or the rank-order sum of the P inputs
// (binary32, one rounding to T, as the vector path).
template <typename T, bool REDUCE>
__device__ __forceinline__ void produce_elem(const SnacArgs& a, const SegGeo& g, int64_t off,
                                             char* dst, int64_t bytes)
{
    using E = typename std::conditional<sizeof(T) == 2, uint16_t, uint32_t>::type;
    const auto ring = ring_rsrc(dst, ceil16(bytes));
    const int64_t n = bytes / static_cast<int64_t>(sizeof(E));
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        E v;
        if (REDUCE) {
            const int64_t e = (g.src_off + off) / static_cast<int64_t>(sizeof(T)) + i;
            float acc = Elem<T>::load(a.src[0], e);
            for (int r = 1; r < a.P; ++r)
                acc = acc + Elem<T>::load(a.src[r], e);
            if (sizeof(T) == 2)
                v = static_cast<E>(f32_to_bf16_bits(acc));
            else
                v = static_cast<E>(__float_as_uint(acc));
        } else {
            v = reinterpret_cast<const E*>(g.src + off)[i];
        }
        ring_store(ring, i * static_cast<int64_t>(sizeof(E)), v);
    }
}

template <typename E>
__device__ __forceinline__ void consume_elem(const SnacArgs& a, const SegGeo& g, const char* src,
                                             int64_t dst_off, int64_t bytes)
{
    const auto ring = ring_rsrc(src, ceil16(bytes));
    const int q0 = g.dst < 0 ? 0 : g.dst;
    const int q1 = g.dst < 0 ? a.P : g.dst + 1;
    const int64_t n = bytes / static_cast<int64_t>(sizeof(E));
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const E v = ring_load<E>(ring, i * static_cast<int64_t>(sizeof(E)));
        for (int q = q0; q < q1; ++q)
            reinterpret_cast<E*>(static_cast<char*>(a.dst[q]) + dst_off)[i] = v;
    }
}

// The two ends of a piece whose streams sit off 16-byte alignment: bytes
// [0, h) and [t0, t0 + tl) of the piece, element by element in one pass
// (one load round trip for both), staged at `dst` in the ring (as
// produce_elem) or consumed from `src` (as consume_elem).
template <typename T, bool REDUCE>
__device__ __forceinline__ void produce_ends(const SnacArgs& a, const SegGeo& g, int64_t off,
                                             char* dst, int64_t h, int64_t t0, int64_t tl)
{
    using E = typename std::conditional<sizeof(T) == 2, uint16_t, uint32_t>::type;
    constexpr int64_t es = sizeof(E);
    const auto ring = ring_rsrc(dst, ceil16(t0 + tl));
    const int64_t nh = h / es, n = nh + tl / es;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const int64_t b = i < nh ? i * es : t0 + (i - nh) * es;      // byte in the piece
        E v;
        if (REDUCE) {
            const int64_t e = (g.src_off + off + b) / static_cast<int64_t>(sizeof(T));
            float acc = Elem<T>::load(a.src[0], e);
            for (int r = 1; r < a.P; ++r)
                acc = acc + Elem<T>::load(a.src[r], e);
            if (sizeof(T) == 2)
                v = static_cast<E>(f32_to_bf16_bits(acc));
            else
                v = static_cast<E>(__float_as_uint(acc));
        } else {
            v = *reinterpret_cast<const E*>(g.src + off + b);
        }
        ring_store(ring, b, v);
    }
}

template <typename E>
__device__ __forceinline__ void consume_ends(const SnacArgs& a, const SegGeo& g, const char* src,
                                             int64_t dst_off, int64_t h, int64_t t0, int64_t tl)
{
    constexpr int64_t es = sizeof(E);
    const auto ring = ring_rsrc(src, ceil16(t0 + tl));
    const int q0 = g.dst < 0 ? 0 : g.dst;
    const int q1 = g.dst < 0 ? a.P : g.dst + 1;
    const int64_t nh = h / es, n = nh + tl / es;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const int64_t b = i < nh ? i * es : t0 + (i - nh) * es;
        const E v = ring_load<E>(ring, b);
        for (int q = q0; q < q1; ++q)
            *reinterpret_cast<E*>(static_cast<char*>(a.dst[q]) + dst_off + b) = v;
    }
}

// The persistent SNAC kernel: UP 16-byte slots per lane in flight while
// staging, UC while consuming, at most MAXT lanes per workgroup (256, or
// 512 for the wide launches, so the default keeps its register budget). T is
// the element type (the reduce stage's, and the unit of the element-wise
// path). Every branch that encloses a barrier depends only on wave-uniform
// values (the ticket and the wait result are read with readfirstlane, the
// segment's path follows from the ticket), and lane 0's work at the end of
// a task (the notify and the next ticket claim) is one divergent region
// closed by a barrier, so all lanes of a workgroup run the same iterations.
template <class Stage, typename T, bool REDUCE, int UP, int UC, int MAXT>
__global__ __launch_bounds__(MAXT) void k_snac(const SnacArgs a)
{
    using E = typename std::conditional<sizeof(T) == 2, uint16_t, uint32_t>::type;
    __shared__ unsigned int s_ticket;
    __shared__ int s_ok;
    touch_arg_lines(&a.src[0], &a.src[8], &a.dst[0], &a.dst[8], &a.ring, &a.chunk_bytes,
                    &a.jitter_seed, &a.cnt[4], &a.elem[0], &a.head[0]);
    const long long t_begin = wall_clock64();
    const int64_t C = a.chunk_bytes;
    // A small call with one workgroup per task (static_tasks) runs task
    // blockIdx.x and no ticket: the grid is dispatched in index order and
    // fits the chip at once, so every task's producers (smaller indices)
    // are running or done. Otherwise tasks are claimed from the ticket.
    const bool fixed = a.static_tasks != 0;
    if (!fixed && threadIdx.x == 0)
        s_ticket = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!fixed)
        __syncthreads();
    int64_t t = fixed ? static_cast<int64_t>(blockIdx.x)
                      : static_cast<unsigned int>(__builtin_amdgcn_readfirstlane(static_cast<int>(s_ticket)));
    unsigned long long* const tr = a.trace;
    long long t_claim = tr ? wall_clock64() : 0;
    while (t < a.ntasks) {
        const Task task = decode_task(a, t);
        const int64_t slot = task.chunk % a.slots;
        const int64_t use = task.chunk / a.slots;             // earlier chunks in this slot
        int s;
        int64_t c;
        chunk_of(a, task.chunk, &s, &c);
        const SegGeo g = seg_geo(a, s);
        const int path = a.elem[s];                // SnacSegPath
        const int d = a.head[s];                   // the sources' offset (SE_VEC, SE_SHIFT)
        const int64_t cbeg = c * C;
        const int64_t clen = (g.bytes - cbeg < C) ? g.bytes - cbeg : C;
        const int64_t pbeg = task.piece * a.piece_bytes;
        int64_t plen = clen - pbeg;
        plen = plen < 0 ? 0 : (plen > a.piece_bytes ? a.piece_bytes : plen);
        char* slotp = a.ring + slot * a.slot_bytes;
        // Stage waits for the slot's previous chunk to be consumed; Consume
        // waits for every piece of its chunk to be staged.
        unsigned long long* const word = a.counts + slot * kFlagStride;
        const unsigned long long target =
            static_cast<unsigned long long>(task.produce ? use : use + 1) * a.pieces;
        const bool ok = wait_at_least(a, word, task.produce, target, t_begin, &s_ok);
        const long long t_wait = tr ? wall_clock64() : 0;
        if (ok) {
            if (!task.produce) {
                jitter(a, t, 1u);
                if (a.jitter_ticks > 0)
                    __syncthreads();
            }
            if (path == SE_ELEM) {
                if (task.produce)
                    produce_elem<T, REDUCE>(a, g, cbeg + pbeg, slotp + pbeg, plen);
                else
                    consume_elem<E>(a, g, slotp + pbeg, g.dst_off + cbeg + pbeg, plen);
            } else if (d == 0) {
                // sources 16-byte aligned: staged at the piece's place
                if (task.produce)
                    Stage::template produce<UP>(a, g, cbeg + pbeg, slotp + pbeg, plen);
                else if (path == SE_SHIFT)
                    consume_shift<kShiftSlots>(a, g, slotp + pbeg, g.dst_off + cbeg + pbeg, plen,
                                               static_cast<int>(sizeof(T)));
                else
                    consume_vec<UC>(a, g, slotp + pbeg, g.dst_off + cbeg + pbeg, plen);
            } else {
                // The segment's sources (and on the vector path every
                // destination) sit d bytes past a 16-byte boundary: the
                // piece's first h = 16 - d bytes (to the boundary) and its
                // last partial vector are staged element by element, the
                // body between them as 16-byte vectors. In the ring the piece
                // starts 112 + d bytes into its place (the slot padding holds
                // the rest), so the body starts on a 128-byte line and the
                // stage's stores fill whole lines.
                char* const rp = slotp + pbeg + 112 + d;
                const int64_t h = plen < kVecBytes - d ? plen : kVecBytes - d;
                const int64_t body = (plen - h) & ~int64_t(kVecBytes - 1);
                const int64_t tail = plen - h - body;
                const int64_t o = cbeg + pbeg;
                // (the body's accesses are issued first, then both ends in
                // one element pass)
                if (task.produce) {
                    Stage::template produce<UP>(a, g, o + h, rp + h, body);
                    produce_ends<T, REDUCE>(a, g, o, rp, h, h + body, tail);
                } else if (path == SE_SHIFT) {
                    // a destination at another offset: the whole piece,
                    // ends included, through the shifted path
                    consume_shift<kShiftSlots>(a, g, rp, g.dst_off + o, plen, static_cast<int>(sizeof(T)));
                } else {
                    consume_vec<UC>(a, g, rp + h, g.dst_off + o + h, body);
                    consume_ends<E>(a, g, rp, g.dst_off + o, h, h + body, tail);
                }
            }
        }
        // Notify: each wave of a producer waits until its write-through
        // stores have completed, so once the barrier is passed the whole
        // piece is agent-visible and the staged count moves with a relaxed
        // increment; a consumer on any XCD that sees the count reads the
        // staged bytes. Releasing the slot publishes no data: the slot loads
        // have already returned (their values were stored before the
        // barrier), so the consumed count moves the same way.
        if (task.produce) {
            wait_vmem();
            jitter(a, t, 2u);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            if (tr) {
                // measurement hook: this task's stamps (ordinary stores)
                unsigned long long* e = tr + 4 * t;
                e[0] = static_cast<unsigned long long>(t_claim);
                e[1] = static_cast<unsigned long long>(t_wait);
                e[2] = static_cast<unsigned long long>(wall_clock64());
                e[3] = static_cast<unsigned long long>(blockIdx.x) |
                       (static_cast<unsigned long long>(task.produce) << 32) |
                       (static_cast<unsigned long long>(!ok) << 33);
            }
            const unsigned long long one = task.produce ? 1ull : kConsumedOne;
            if (fixed) {
                // A small call's workgroup ends with its one task. Its count
                // is a returning add, and the task that brings both of the
                // slot's counts to their final values (every piece of every
                // chunk the slot holds, staged and consumed) clears the word
                // for the next call: no other task of this call touches it
                // again. Every task counts, also one whose wait gave up, so
                // the word always reaches its final value.
                const unsigned long long uses =
                    static_cast<unsigned long long>((a.nchunks - 1 - slot) / a.slots + 1);
                const unsigned long long fin = uses * static_cast<unsigned long long>(a.pieces) *
                                               (kConsumedOne + 1ull);
                if (!task.produce && ok && uses == 1 && a.pieces == 1) {
                    // The slot's only consumer, past its wait: the only
                    // producer has counted, so the word is clear to reset
                    // without the add's round trip.
                    __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else if (__hip_atomic_fetch_add(word, one, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT) + one == fin) {
                    __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            } else if (ok) {
                flag_add_relaxed(word, one);
            }
            if (!fixed)
                s_ticket = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        t = fixed ? a.ntasks
                  : static_cast<unsigned int>(__builtin_amdgcn_readfirstlane(static_cast<int>(s_ticket)));
        if (tr)
            t_claim = wall_clock64();
    }
    // A small call has cleared its slot words in its tasks and used neither
    // the ticket nor the finished-workgroup count.
    if (fixed)
        return;
    // Every workgroup counts itself out; the last one clears the ticket, the
    // slot words and the count for the next staged call on this device,
    // so a call is one launch and a captured graph replays from a clean
    // state. Lane 0 made all of this workgroup's counter updates; it waits
    // until they have completed before counting out, and the last workgroup
    // clears only after its count returned, so every update of this call
    // precedes the clearing. The error word is kept for the host.
    // Only the slots this call used (chunk q takes slot q mod D) have moved;
    // the others are still zero from the call that last used them. The last
    // workgroup clears them one per lane.
    if (threadIdx.x == 0) {
        wait_vmem();
        const unsigned int prev =
            __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_ok = prev == gridDim.x - 1 ? 1 : 0;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_ok) != 0) {
        const int used = static_cast<int>(a.nchunks < a.slots ? a.nchunks : a.slots);
        for (int i = threadIdx.x; i < used; i += blockDim.x)
            __hip_atomic_store(a.counts + i * kFlagStride, 0ull, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (threadIdx.x == 0) {
            __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---- calls that stage each chunk once: the tagged ring ------------------
// A call whose ring would hold every chunk (no slot is reused; one
// workgroup per task) and each of whose segments has its streams at one
// offset from 16-byte alignment hands off through tagged words instead of
// slot counts. Its piece's place in the tag region holds one
// 64-bit pair per staged 4-byte word: the word in the low half, the call's
// sequence number in the high half, written by one agent-scope 64-bit store
// (a naturally aligned 64-bit access is single-copy atomic, and the
// agent-scope policy writes it through the producer's L2). The notify is
// the tag itself: a consumer that loads a pair carrying this call's number
// (agent scope: never a stale L2 line) has that word. The producer neither
// waits for its stores nor counts; the consumer polls its own pairs instead
// of a count, and reads no ring after it. Each consumer then clears the
// pairs it took, so the region keeps no pair with the call's number: a
// replay of a captured call, which keeps its number, waits for its own
// producers. Pairs that a consumer which gave up left behind carry that
// call's number, which no later call takes until the numbers start over,
// when the host clears the region (launch_clear_tags).
//
// A segment whose streams all sit d bytes past a 16-byte boundary (its
// pieces too: chunks and pieces are multiples of 16 bytes) is staged in the
// aligned 16-byte vectors that enclose each piece, vector v holding piece
// bytes [16 v - d, 16 v - d + 16); the consumer writes only the piece's
// bytes (element by element in the first and last vector). A load of an
// enclosing vector stays in the 16-byte block of a segment byte.
// Pairs are laid out so that one instruction of a wave moves 64 adjacent
// pairs: word j of vector v of a piece is pair 256 * (v / 64) + 64 * j +
// v mod 64 of the piece's place (tag_place pairs: a piece is a multiple of
// 1 KiB, and the place has one more group of 64 vectors when a segment sits
// off alignment, so a piece's pairs stay inside its own place). Each wave polls on its own, with no
// barrier inside a loop; a wave's loop exits on a ballot over its lanes, so
// its lanes leave together. Waits are bounded as in the persistent kernel.
constexpr int kTagVecs = 2;   // 16-byte vectors per lane per round
// A waiting lane polls all four words of its vectors while the call has at
// most this many consumer tasks; with more, it polls only each vector's
// first word and loads the other three once that word carries the tag, so
// that the polls of many waiting consumers do not crowd the producers'
// stores. Measured on MI355X, back to back, all words / first word: the
// staged AllGather of 8 x 8 KiB 4.93 / 5.16 us, AllReduce of 8 x 16 KiB
// 4.98 / 5.49 us (16 consumers); AllGather of 8 x 64 KiB 6.10 / 5.98 us
// (64), of 8 x 128 KiB 7.3 / 6.78 us (128).
constexpr int64_t kTagPollAllTasks = 32;

__device__ __forceinline__ int64_t tag_pair(int64_t v, int j)
{
    return ((v >> 6) << 8) + (j << 6) + (v & 63);
}

template <class Stage, int MAXT>
__global__ __launch_bounds__(MAXT) void k_snac_tagged(const SnacArgs a)
{
    touch_arg_lines(&a.src[0], &a.src[8], &a.dst[0], &a.dst[8], &a.ring, &a.chunk_bytes,
                    &a.jitter_seed, &a.cnt[4], &a.elem[0], &a.head[0]);
    const long long t_begin = wall_clock64();
    const int64_t t = blockIdx.x;
    if (t >= a.ntasks)
        return;
    const Task task = decode_task(a, t);
    int s;
    int64_t c;
    chunk_of(a, task.chunk, &s, &c);
    const SegGeo g = seg_geo(a, s);
    const int64_t C = a.chunk_bytes;
    const int64_t cbeg = c * C;
    const int64_t clen = (g.bytes - cbeg < C) ? g.bytes - cbeg : C;
    const int64_t pbeg = task.piece * a.piece_bytes;
    int64_t plen = clen - pbeg;
    plen = plen < 0 ? 0 : (plen > a.piece_bytes ? a.piece_bytes : plen);
    unsigned long long* const pairs = a.tags + (task.chunk * a.pieces + task.piece) * a.tag_place;
    const int d = a.head[s];                   // the segment's offset from 16-byte alignment
    const uint32_t seq = a.seq;
    const unsigned long long tag = static_cast<unsigned long long>(seq) << 32;
    if (a.jitter_ticks > 0) {
        jitter(a, t, task.produce ? 2u : 1u);
        __syncthreads();
    }
    const int lane = threadIdx.x;
    const int64_t nthr = blockDim.x;
    // aligned vectors enclosing the piece (none for an empty piece past a
    // segment's end); the first and last are staged whole and only their
    // piece bytes are written out
    const int64_t nv = plen > 0 ? (d + plen + kVecBytes - 1) / kVecBytes : 0;
    bool ok = true;
    long long t_wait = t_begin;
    if (task.produce) {
        for (int64_t v0 = 0; v0 < nv; v0 += nthr * kTagVecs) {
            u32x4 x[kTagVecs];
#pragma unroll
            for (int u = 0; u < kTagVecs; ++u) {
                const int64_t v = v0 + u * nthr + lane;
                if (v < nv)
                    x[u] = Stage::stage_vec(a, g, cbeg + pbeg - d + v * kVecBytes);
            }
#pragma unroll
            for (int u = 0; u < kTagVecs; ++u) {
                const int64_t v = v0 + u * nthr + lane;
                if (v < nv) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        __hip_atomic_store(pairs + tag_pair(v, j), tag | x[u][j], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    } else {
        const bool nt = a.nt_store != 0;
        const int q0 = g.dst < 0 ? 0 : g.dst;
        const int q1 = g.dst < 0 ? a.P : g.dst + 1;
        const int64_t dst_off = g.dst_off + cbeg + pbeg - d;     // 16-byte aligned
        const bool all_words = a.nchunks * a.pieces <= kTagPollAllTasks;
        for (int64_t v0 = 0; v0 < nv && ok; v0 += nthr * kTagVecs) {
            unsigned long long w[kTagVecs][4];
#pragma unroll
            for (int u = 0; u < kTagVecs; ++u) {
                const int64_t v = v0 + u * nthr + lane;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w[u][j] = v >= nv ? tag
                              : (j == 0 || all_words)
                                  ? __hip_atomic_load(pairs + tag_pair(v, j), __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                                  : 0ull;    // not yet loaded (no call's tag is 0)
            }
            long long w0 = 0;
            for (unsigned int it = 0;; ++it) {
                bool ready = true;
#pragma unroll
                for (int u = 0; u < kTagVecs; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        ready = ready && static_cast<uint32_t>(w[u][j] >> 32) == seq;
                if (__builtin_amdgcn_ballot_w64(!ready) == 0)
                    break;
                if (it == 0)
                    w0 = wall_clock64();
                if (it < 8)
                    __builtin_amdgcn_s_sleep(1);
                else
                    __builtin_amdgcn_s_sleep(8);
                if ((it & 15u) == 15u) {
                    const long long now = wall_clock64();
                    const uint32_t err = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(
                        __hip_atomic_load(a.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))));
                    if (err == seq || now - w0 > a.wait_ticks || now - t_begin > a.budget_ticks) {
                        if ((threadIdx.x & 63) == 0)
                            __hip_atomic_store(a.error, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        ok = false;
                        break;
                    }
                }
#pragma unroll
                for (int u = 0; u < kTagVecs; ++u) {
                    const int64_t v = v0 + u * nthr + lane;
                    const bool first = static_cast<uint32_t>(w[u][0] >> 32) == seq;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (v < nv && static_cast<uint32_t>(w[u][j] >> 32) != seq &&
                            (j == 0 || first || all_words))
                            w[u][j] = __hip_atomic_load(pairs + tag_pair(v, j), __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            if (!ok)
                break;
            if (v0 == 0)
                t_wait = wall_clock64();
#pragma unroll
            for (int u = 0; u < kTagVecs; ++u) {
                const int64_t v = v0 + u * nthr + lane;
                if (v >= nv)
                    continue;
                const u32x4 x = {static_cast<uint32_t>(w[u][0]), static_cast<uint32_t>(w[u][1]),
                                 static_cast<uint32_t>(w[u][2]), static_cast<uint32_t>(w[u][3])};
                const int64_t o = v * kVecBytes;
                // whole vectors here; the piece's partial first and last
                // vectors below, one destination per lane
                if (v != 0 && o + kVecBytes <= d + plen) {
                    for (int q = q0; q < q1; ++q)
                        st16(static_cast<char*>(a.dst[q]) + dst_off, static_cast<uint32_t>(o), x, nt);
                } else if (v == 0 && d == 0 && kVecBytes <= plen) {
                    for (int q = q0; q < q1; ++q)
                        st16(static_cast<char*>(a.dst[q]) + dst_off, static_cast<uint32_t>(o), x, nt);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    __hip_atomic_store(pairs + tag_pair(v, j), 0ull, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            // The piece's partial vectors (its first when d > 0, its last
            // when it ends inside a vector): the wave holding one reads it
            // from its owner lane, and lane i writes destination q0 + i
            // (a few element stores each, in parallel over the outputs).
            const int64_t round = nthr * kTagVecs;
            for (int e = 0; e < 2; ++e) {
                const int64_t pv = e == 0 ? 0 : nv - 1;
                const int p0 = pv == 0 ? d : 0;
                const int64_t end = d + plen - pv * kVecBytes;
                const int p1 = end < kVecBytes ? static_cast<int>(end) : static_cast<int>(kVecBytes);
                if ((p0 == 0 && p1 == kVecBytes) || (e == 1 && pv == 0) || pv < v0 || pv >= v0 + round)
                    continue;                              // whole, already done, or another round
                const int64_t idx = pv - v0;               // = u * nthr + owner
                const int pu = static_cast<int>(idx / nthr);
                const int owner = static_cast<int>(idx - static_cast<int64_t>(pu) * nthr);
                if ((threadIdx.x >> 6) != (owner >> 6))
                    continue;                              // (wave-uniform)
                u32x4 x = {0, 0, 0, 0};
#pragma unroll
                for (int u = 0; u < kTagVecs; ++u) {
                    if (u == pu) {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            x[j] = static_cast<uint32_t>(__builtin_amdgcn_readlane(
                                static_cast<int>(static_cast<uint32_t>(w[u][j])), owner & 63));
                    }
                }
                // lane i takes destination q0 + i; each pointer is made
                // wave-uniform first, so it is read with scalar loads and
                // selected per lane (the argument array is never indexed by
                // a vector register). Measured on MI355X, back to back with
                // every buffer one bf16 element off: the staged AllGather
                // of 8 x 8 KiB 9.9 -> 6.7 us and AllReduce of 8 x 1 KiB
                // 8.3 -> 5.6 us, against one lane writing every output.
                uint64_t dq = 0;
                for (int q = q0; q < q1; ++q) {
                    const uint64_t pq = reinterpret_cast<uint64_t>(a.dst[q]);
                    const uint64_t u = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(pq))) |
                                       (static_cast<uint64_t>(static_cast<uint32_t>(
                                            __builtin_amdgcn_readfirstlane(static_cast<int>(pq >> 32))))
                                        << 32);
                    dq = (threadIdx.x & 63) == q - q0 ? u : dq;
                }
                if (dq)
                    store_slot_part(reinterpret_cast<char*>(dq) + dst_off + pv * kVecBytes, x, p0, p1, 2);
            }
        }
    }
    if (a.trace) {
        // measurement hook: this task's stamps, taken when every wave is done
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long* e = a.trace + 4 * t;
            e[0] = static_cast<unsigned long long>(t_begin);
            e[1] = static_cast<unsigned long long>(t_wait);
            e[2] = static_cast<unsigned long long>(wall_clock64());
            e[3] = static_cast<unsigned long long>(blockIdx.x) |
                   (static_cast<unsigned long long>(task.produce) << 32) |
                   (static_cast<unsigned long long>(!ok) << 33);
        }
    }
}

// The reducing stage keeps P * UP loads in flight per lane: UP = 2 up to
// P = 8, 1 for more inputs.
template <typename T, int MAXT>
hipError_t launch_reduce_t(const SnacArgs& a, dim3 grid, dim3 block, hipStream_t stream)
{
    switch (a.P) {
#define ATOM_SNAC_RED_CASE(PP)                                                                  \
    case PP:                                                                                    \
        k_snac<StageReduce<T, PP>, T, true, (PP <= 8 ? 2 : 1), 8, MAXT><<<grid, block, 0, stream>>>(a); \
        break;
    ATOM_SNAC_RED_CASE(1) ATOM_SNAC_RED_CASE(2) ATOM_SNAC_RED_CASE(3) ATOM_SNAC_RED_CASE(4)
    ATOM_SNAC_RED_CASE(5) ATOM_SNAC_RED_CASE(6) ATOM_SNAC_RED_CASE(7) ATOM_SNAC_RED_CASE(8)
    ATOM_SNAC_RED_CASE(9) ATOM_SNAC_RED_CASE(10) ATOM_SNAC_RED_CASE(11) ATOM_SNAC_RED_CASE(12)
    ATOM_SNAC_RED_CASE(13) ATOM_SNAC_RED_CASE(14) ATOM_SNAC_RED_CASE(15) ATOM_SNAC_RED_CASE(16)
#undef ATOM_SNAC_RED_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The tagged kernels are built for up to 512 lanes (the staged default).
template <typename T>
hipError_t launch_tagged_reduce_t(const SnacArgs& a, dim3 grid, dim3 block, hipStream_t stream)
{
    switch (a.P) {
#define ATOM_SNAC_TAG_CASE(PP)                                                                  \
    case PP: k_snac_tagged<StageReduce<T, PP>, 512><<<grid, block, 0, stream>>>(a); break;
    ATOM_SNAC_TAG_CASE(1) ATOM_SNAC_TAG_CASE(2) ATOM_SNAC_TAG_CASE(3) ATOM_SNAC_TAG_CASE(4)
    ATOM_SNAC_TAG_CASE(5) ATOM_SNAC_TAG_CASE(6) ATOM_SNAC_TAG_CASE(7) ATOM_SNAC_TAG_CASE(8)
    ATOM_SNAC_TAG_CASE(9) ATOM_SNAC_TAG_CASE(10) ATOM_SNAC_TAG_CASE(11) ATOM_SNAC_TAG_CASE(12)
    ATOM_SNAC_TAG_CASE(13) ATOM_SNAC_TAG_CASE(14) ATOM_SNAC_TAG_CASE(15) ATOM_SNAC_TAG_CASE(16)
#undef ATOM_SNAC_TAG_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int MAXT>
hipError_t launch_copy_t(const SnacArgs& a, int U, dim3 grid, dim3 block, hipStream_t stream)
{
    switch (U) {
#define ATOM_SNAC_COPY_CASE(UU)                                                              \
    case UU: k_snac<StageCopy, T, false, UU, UU, MAXT><<<grid, block, 0, stream>>>(a); break;
    ATOM_SNAC_COPY_CASE(1) ATOM_SNAC_COPY_CASE(2) ATOM_SNAC_COPY_CASE(4) ATOM_SNAC_COPY_CASE(8)
#undef ATOM_SNAC_COPY_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---- the fixed workspace of atom_collective_noalloc ---------------------
// Flags (the slot count words, the ticket, the error word and the
// finished-workgroup count, each on its own 256-byte line, as in the
// allocated workspace), the tagged ring (kTagBytes), then a
// ring of kStaticRingBytes. Each device holds its own copy from the
// library's load until the process ends.
constexpr int64_t kFlagLine = kFlagStride * sizeof(unsigned long long);
constexpr int64_t kStaticFlagBytes = 64 << 10;
static_assert((kMaxSlots + 3) * kFlagLine <= kStaticFlagBytes, "flags do not fit");
// The ring part also holds each slot's padding (kSlotPad), so that a ring of
// kStaticRingBytes of chunks fits at any depth up to kMaxSlots.
constexpr int64_t kStaticRingAlloc = kStaticRingBytes + kMaxSlots * kSlotPad;
static __device__ __align__(256) char scratch[kStaticFlagBytes + kTagBytes + kStaticRingAlloc];

__global__ void k_clear_words(unsigned long long* p, int64_t n)
{
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = 0;
}

std::mutex g_static_mutex;
Workspace g_static_ws[kMaxDevices];   // .ring == NULL until set up on that device

}  // namespace

atom_status static_workspace(hipStream_t stream, Workspace** out, hipError_t* hip_err)
{
    int dev = 0;
    if ((*hip_err = hipGetDevice(&dev)) != hipSuccess)
        return ATOM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return ATOM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_static_mutex);
    Workspace& ws = g_static_ws[dev];
    if (!ws.ring) {
        // The array's name is a host-side stand-in: its device address on
        // this device comes from the runtime, and only that address is used.
        char* ptr = nullptr;
        if ((*hip_err = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
            return ATOM_ERR_HIP;
        if (!ptr)
            return ATOM_ERR_UNSUPPORTED;
        int khz = 0;
        if ((*hip_err = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess)
            return ATOM_ERR_HIP;
        if (khz <= 0)
            return ATOM_ERR_UNSUPPORTED;
        k_clear_words<<<64, 256, 0, stream>>>(reinterpret_cast<unsigned long long*>(ptr),
                                              (kStaticFlagBytes + kTagBytes) / 8);
        if ((*hip_err = hipGetLastError()) != hipSuccess)
            return ATOM_ERR_HIP;
        ws.wall_khz = khz;
        ws.counts = reinterpret_cast<unsigned long long*>(ptr);
        ws.ticket = reinterpret_cast<unsigned int*>(ptr + kMaxSlots * kFlagLine);
        ws.error = reinterpret_cast<unsigned int*>(ptr + (kMaxSlots + 1) * kFlagLine);
        ws.done = reinterpret_cast<unsigned int*>(ptr + (kMaxSlots + 2) * kFlagLine);
        ws.tags = reinterpret_cast<unsigned long long*>(ptr + kStaticFlagBytes);
        ws.ring_bytes = kStaticRingAlloc;
        ws.ring = ptr + kStaticFlagBytes + kTagBytes;
    }
    if (++ws.seq == 0) {
        // the numbers start over: no stale pair may carry one of them
        ws.seq = 1;
        if ((*hip_err = launch_clear_tags(ws, stream)) != hipSuccess)
            return ATOM_ERR_HIP;
    }
    *out = &ws;
    return ATOM_OK;
}

hipError_t launch_clear_tags(const Workspace& ws, hipStream_t stream)
{
    if (!ws.tags)
        return hipErrorInvalidValue;
    k_clear_words<<<64, 256, 0, stream>>>(ws.tags, kTagBytes / 8);
    return hipGetLastError();
}

unsigned int* static_error_word(int dev)
{
    if (dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_static_mutex);
    return g_static_ws[dev].error;
}

hipError_t launch_snac(const Plan& p, const Workspace& ws, uint32_t seq, hipStream_t stream)
{
    if ((p.exec != EX_SNAC_COPY && p.exec != EX_SNAC_REDUCE) || !ws.ring ||
        ws.ring_bytes < p.ring_bytes || p.grid < 1 || p.sa.slots < 1 || p.sa.slots > kMaxSlots ||
        p.sa.pieces < 1 || p.sa.lead < 1 || p.sa.lead > p.sa.slots || p.sa.P < 1 ||
        p.sa.P > kMaxRanks || p.sa.nseg < 1 ||
        p.sa.nseg > kMaxSegs || ws.wall_khz <= 0 || p.wg < 64 || p.wg > 512 || p.wg % 64 != 0 ||
        !ws.done || seq == 0)
        return hipErrorInvalidValue;
    if (p.sa.tagged && (!ws.tags || !p.sa.static_tasks || p.grid != p.sa.ntasks ||
                        p.sa.piece_bytes % 1024 != 0 || p.sa.chunk_bytes % p.sa.piece_bytes != 0 ||
                        p.sa.tag_place < p.sa.piece_bytes / 4 ||
                        p.sa.nchunks * p.sa.pieces * p.sa.tag_place * 8 > kTagBytes))
        return hipErrorInvalidValue;
    SnacArgs a = p.sa;
    a.ring = ws.ring;
    a.tags = ws.tags;
    a.counts = ws.counts;
    a.ticket = ws.ticket;
    a.error = ws.error;
    a.done = ws.done;
    a.seq = seq;
    // Bounds in device-clock ticks (kHz x ms): the planned wait bound (1 s
    // unless the caller shortened it) and ~10 s per workgroup; the test
    // hook's delay likewise.
    a.wait_ticks = std::max<int64_t>(1, static_cast<int64_t>(ws.wall_khz) * p.sa.wait_ticks / 1000);
    a.budget_ticks = static_cast<int64_t>(ws.wall_khz) * 10000;
    a.jitter_ticks = static_cast<int64_t>(ws.wall_khz) * p.sa.jitter_ticks / 1000;
    const dim3 grid(static_cast<unsigned>(p.grid)), block(static_cast<unsigned>(p.wg));
    const bool wide = p.wg > 256;
    const bool bf = p.dtype == DT_BF16;
    if (a.tagged) {
        if (p.exec == EX_SNAC_COPY) {
            k_snac_tagged<StageCopy, 512><<<grid, block, 0, stream>>>(a);
            return hipGetLastError();
        }
        return bf ? launch_tagged_reduce_t<uint16_t>(a, grid, block, stream)
                  : launch_tagged_reduce_t<float>(a, grid, block, stream);
    }
    if (p.exec == EX_SNAC_COPY) {
        if (bf)
            return wide ? launch_copy_t<uint16_t, 512>(a, p.U, grid, block, stream)
                        : launch_copy_t<uint16_t, 256>(a, p.U, grid, block, stream);
        return wide ? launch_copy_t<float, 512>(a, p.U, grid, block, stream)
                    : launch_copy_t<float, 256>(a, p.U, grid, block, stream);
    }
    if (bf)
        return wide ? launch_reduce_t<uint16_t, 512>(a, grid, block, stream)
                    : launch_reduce_t<uint16_t, 256>(a, grid, block, stream);
    return wide ? launch_reduce_t<float, 512>(a, grid, block, stream)
                : launch_reduce_t<float, 256>(a, grid, block, stream);
}

}  // namespace atom
