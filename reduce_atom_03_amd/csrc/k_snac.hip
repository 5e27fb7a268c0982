// k_snac.hip -- SNAC (Stage, Notify, And Consume) on one gfx950 device.
//
// "Purlin: Separating Orchestration from the Datapath of Collectives"
// (arXiv 2609.36954): the abstract introduces SNAC as the orchestration
// shared by every collective, derived from the layouts; Figure 6 shows ranks
// staging chunks incrementally while consumers gather them; Table 3 sizes a
// chunk as the bandwidth-delay product; Figures 9 and 10 contrast ordinary
// buffers (staged) with peer-accessible ones (zero staging).
//
// On one device the P ranks are P buffers and the hand-off between a
// producer and its consumers crosses workgroups (and XCDs, each with its own
// L2) through device memory:
//   Stage   a producer workgroup copies one piece of a chunk of partition k
//           into a slot of the staging ring with agent-coherent stores;
//   Notify  once every wave's stores have completed it adds 1 to the
//           slot's `ready` counter;
//   Consume a consumer workgroup waits for `ready` == all pieces of the
//           chunk, reads one piece from the slot with agent-coherent loads,
//           writes it to every output (AllGather fan-out) and adds 1 to the
//           slot's `freed` counter, which the producer of the chunk D
//           places later waits for before reuse.
// The ring is never touched by ordinary (L2-cached) accesses, so no task
// needs an L2 write-back or invalidation.
//
// Tasks are claimed from one atomic ticket in an order where every task
// depends only on tasks with smaller tickets: producers of chunks 0..D-1,
// then for each later chunk q the consumers of chunk q-D followed by the
// producers of chunk q, then the consumers of the last D chunks. A claimed
// ticket belongs to a running workgroup, so the lowest unfinished task can
// always proceed: no deadlock for any grid size or occupancy. Every wait is
// bounded; on expiry the error word is set, the task is dropped, and later
// waits give up at once, so the grid always drains.
#include <algorithm>

#include "atom_dev.hpp"
#include "launch.hpp"

namespace atom {

namespace {

struct Task {
    bool produce;
    int64_t chunk;
    int64_t piece;
};

__device__ __forceinline__ Task decode_task(const SnacArgs& a, int64_t t)
{
    const int64_t G = a.pieces, D = a.slots, Q = a.nchunks;
    const int64_t warm = (Q < D ? Q : D) * G;              // producers of chunks 0..D-1
    const int64_t mid = (Q > D ? Q - D : 0) * 2 * G;       // [consume q-D, produce q]
    Task k;
    if (t < warm) {
        k.produce = true;
        k.chunk = t / G;
        k.piece = t - k.chunk * G;
    } else if (t < warm + mid) {
        const int64_t u = t - warm;
        const int64_t q = D + u / (2 * G);
        const int64_t w = u - (q - D) * 2 * G;
        k.produce = w >= G;
        k.chunk = k.produce ? q : q - D;
        k.piece = k.produce ? w - G : w;
    } else {
        const int64_t u = t - warm - mid;
        k.produce = false;
        k.chunk = (Q > D ? Q - D : 0) + u / G;
        k.piece = u - (u / G) * G;
    }
    return k;
}

// Lane 0 waits until *flag >= target, bounded in wall-clock time (the
// per-wait bound and the workgroup's whole-kernel budget, both in ticks of
// the constant-rate device clock). The barrier then holds every wave until
// the count was seen, so the waves' ring loads are issued after it. The
// result is made wave-uniform with readfirstlane so every branch on it is
// uniform. Returns false when the wait gave up (a timeout here or
// elsewhere).
__device__ __forceinline__ bool wait_at_least(const SnacArgs& a, const unsigned long long* flag,
                                              unsigned long long target, long long t_begin,
                                              int* s_ok)
{
    if (threadIdx.x == 0) {
        int ok = 1;
        if (flag_load_relaxed(flag) < target) {
            const long long w0 = wall_clock64();
            unsigned int it = 0;
            while (flag_load_relaxed(flag) < target) {
                // Back off: waiting workgroups poll one counter line, and a
                // poll that misses costs the producers memory bandwidth.
                if (it < 8)
                    __builtin_amdgcn_s_sleep(2);
                else
                    __builtin_amdgcn_s_sleep(16);
                if ((++it & 15u) == 0) {
                    const long long now = wall_clock64();
                    if (__hip_atomic_load(a.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
                        now - w0 > a.wait_ticks || now - t_begin > a.budget_ticks) {
                        __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Stage producers: fill `bytes` bytes (a multiple of 16) of a ring slot.
// Copy: partition k of its own input (AllGather).
struct StageCopy {
    template <int U>
    __device__ static void produce(const SnacArgs& a, int k, int64_t off, char* dst, int64_t bytes)
    {
        const char* src = static_cast<const char*>(a.src[k]) + off;
        const auto ring = ring_rsrc(dst, bytes);
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

// Reduce: partition k summed over the P inputs in rank order, rounded once
// (the ReduceScatter half of the composed AllReduce, Figure 6).
template <typename T, int P>
struct StageReduce {
    template <int U>
    __device__ static void produce(const SnacArgs& a, int k, int64_t off, char* dst, int64_t bytes)
    {
        const int64_t base = static_cast<int64_t>(k) * a.part_bytes + off;
        const auto ring = ring_rsrc(dst, bytes);
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

// Consume: one piece from the slot to every output (AllGather fan-out).
template <int U>
__device__ __forceinline__ void fan_out(const SnacArgs& a, const char* src, int64_t dst_off, int64_t bytes)
{
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const bool nt = a.nt_store != 0;
    const auto ring = ring_rsrc(src, bytes);
    const int64_t step = static_cast<int64_t>(nthr) * U * kVecBytes;
    for (int64_t b0 = 0; b0 < bytes; b0 += step) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t o = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
            if (o < bytes)
                x[u] = ld16_agent(ring, o);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t off = static_cast<uint32_t>(u * nthr + lane) * kVecBytes;
            if (b0 + off < bytes)
                for (int q = 0; q < a.P; ++q)
                    st16(static_cast<char*>(a.dst[q]) + dst_off + b0, off, x[u], nt);
        }
    }
}

// The persistent SNAC kernel: UP 16-byte slots per lane in flight while
// staging, UC while fanning out, at most MAXT lanes per workgroup (256, or
// 512 for the wide launches, so the default keeps its register budget). Every branch that encloses a barrier depends
// only on wave-uniform values (the ticket and the wait result are read with
// readfirstlane), and lane 0's work at the end of a task (the notify and the
// next ticket claim) is one divergent region closed by a barrier, so all
// lanes of a workgroup run the same iterations.
template <class Stage, int UP, int UC, int MAXT>
__global__ __launch_bounds__(MAXT) void k_snac(const SnacArgs a)
{
    __shared__ unsigned int s_ticket;
    __shared__ int s_ok;
    const long long t_begin = wall_clock64();
    const int64_t S = a.part_bytes;
    const int64_t C = a.chunk_bytes;
    if (threadIdx.x == 0)
        s_ticket = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int64_t t = static_cast<unsigned int>(__builtin_amdgcn_readfirstlane(static_cast<int>(s_ticket)));
    while (t < a.ntasks) {
        const Task task = decode_task(a, t);
        const int64_t slot = task.chunk % a.slots;
        const int64_t use = task.chunk / a.slots;             // earlier chunks in this slot
        const int k = static_cast<int>(task.chunk % a.P);     // partitions interleave
        const int64_t c = task.chunk / a.P;                   // chunk index within partition k
        const int64_t cbeg = c * C;
        const int64_t clen = (S - cbeg < C) ? S - cbeg : C;
        const int64_t pbeg = task.piece * a.piece_bytes;
        int64_t plen = clen - pbeg;
        plen = plen < 0 ? 0 : (plen > a.piece_bytes ? a.piece_bytes : plen);
        char* slotp = a.ring + slot * C;
        // Stage waits for the slot's previous chunk to be consumed; Consume
        // waits for every piece of its chunk to be staged.
        const unsigned long long* wflag = (task.produce ? a.freed : a.ready) + slot * kFlagStride;
        const unsigned long long target =
            static_cast<unsigned long long>(task.produce ? use : use + 1) * a.pieces;
        const bool ok = wait_at_least(a, wflag, target, t_begin, &s_ok);
        if (ok) {
            if (task.produce) {
                Stage::template produce<UP>(a, k, cbeg + pbeg, slotp + pbeg, plen);
            } else {
                fan_out<UC>(a, slotp + pbeg, static_cast<int64_t>(k) * S + cbeg + pbeg, plen);
            }
        }
        // Notify: each wave of a producer waits until its write-through
        // stores have completed, so once the barrier is passed the whole
        // piece is agent-visible and `ready` moves with a relaxed increment;
        // a consumer on any XCD that sees the count reads the staged bytes.
        // Releasing the slot publishes no data: the slot loads have already
        // returned (their values were stored before the barrier), so `freed`
        // moves the same way.
        if (task.produce)
            wait_vmem();
        __syncthreads();
        if (threadIdx.x == 0) {
            if (ok)
                flag_add_relaxed((task.produce ? a.ready : a.freed) + slot * kFlagStride, 1ull);
            s_ticket = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        t = static_cast<unsigned int>(__builtin_amdgcn_readfirstlane(static_cast<int>(s_ticket)));
    }
    // Every workgroup counts itself out; the last one clears the ticket, the
    // slot counters and the count for the next staged call on this device,
    // so a call is one launch and a captured graph replays from a clean
    // state. Lane 0 made all of this workgroup's counter updates; it waits
    // until they have completed before counting out, and the last workgroup
    // clears only after its count returned, so every update of this call
    // precedes the clearing. The error word is kept for the host.
    if (threadIdx.x == 0) {
        wait_vmem();
        const unsigned int prev =
            __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == gridDim.x - 1) {
            for (int s = 0; s < a.slots; ++s) {
                __hip_atomic_store(a.ready + s * kFlagStride, 0ull, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(a.freed + s * kFlagStride, 0ull, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The reducing stage keeps P * UP loads in flight per lane: UP = 2 up to
// P = 8, 1 for more inputs.
template <typename T, int MAXT>
hipError_t launch_ar_t(const SnacArgs& a, dim3 grid, dim3 block, hipStream_t stream)
{
    switch (a.P) {
#define ATOM_SNAC_AR_CASE(PP) \
    case PP: k_snac<StageReduce<T, PP>, (PP <= 8 ? 2 : 1), 8, MAXT><<<grid, block, 0, stream>>>(a); break;
    ATOM_SNAC_AR_CASE(1) ATOM_SNAC_AR_CASE(2) ATOM_SNAC_AR_CASE(3) ATOM_SNAC_AR_CASE(4)
    ATOM_SNAC_AR_CASE(5) ATOM_SNAC_AR_CASE(6) ATOM_SNAC_AR_CASE(7) ATOM_SNAC_AR_CASE(8)
    ATOM_SNAC_AR_CASE(9) ATOM_SNAC_AR_CASE(10) ATOM_SNAC_AR_CASE(11) ATOM_SNAC_AR_CASE(12)
    ATOM_SNAC_AR_CASE(13) ATOM_SNAC_AR_CASE(14) ATOM_SNAC_AR_CASE(15) ATOM_SNAC_AR_CASE(16)
#undef ATOM_SNAC_AR_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_snac(const Plan& p, const Workspace& ws, hipStream_t stream)
{
    if ((p.exec != EX_SNAC_AG && p.exec != EX_SNAC_AR) || !ws.ring || ws.ring_bytes < p.ring_bytes ||
        p.grid < 1 || p.sa.slots < 1 || p.sa.slots > kMaxSlots || p.sa.pieces < 1 || p.sa.P < 1 ||
        p.sa.P > kMaxRanks || ws.wall_khz <= 0 || p.wg < 64 || p.wg > 512 || p.wg % 64 != 0 ||
        !ws.done)
        return hipErrorInvalidValue;
    SnacArgs a = p.sa;
    a.ring = ws.ring;
    a.ready = ws.ready;
    a.freed = ws.freed;
    a.ticket = ws.ticket;
    a.error = ws.error;
    a.done = ws.done;
    // Bounds in device-clock ticks (kHz x ms): the planned wait bound (1 s
    // unless the caller shortened it) and ~10 s per workgroup.
    a.wait_ticks = std::max<int64_t>(1, static_cast<int64_t>(ws.wall_khz) * p.sa.wait_ticks / 1000);
    a.budget_ticks = static_cast<int64_t>(ws.wall_khz) * 10000;
    const dim3 grid(static_cast<unsigned>(p.grid)), block(static_cast<unsigned>(p.wg));
    const bool wide = p.wg > 256;
    if (p.exec == EX_SNAC_AG) {
#define ATOM_SNAC_AG_CASE(UU)                                                              \
    case UU:                                                                               \
        if (wide)                                                                          \
            k_snac<StageCopy, UU, UU, 512><<<grid, block, 0, stream>>>(a);                 \
        else                                                                               \
            k_snac<StageCopy, UU, UU, 256><<<grid, block, 0, stream>>>(a);                 \
        break;
        switch (p.U) {
        ATOM_SNAC_AG_CASE(1) ATOM_SNAC_AG_CASE(2) ATOM_SNAC_AG_CASE(4) ATOM_SNAC_AG_CASE(8)
        default: return hipErrorInvalidValue;
        }
#undef ATOM_SNAC_AG_CASE
        return hipGetLastError();
    }
    if (p.dtype == DT_BF16)
        return wide ? launch_ar_t<uint16_t, 512>(a, grid, block, stream)
                    : launch_ar_t<uint16_t, 256>(a, grid, block, stream);
    return wide ? launch_ar_t<float, 512>(a, grid, block, stream)
                : launch_ar_t<float, 256>(a, grid, block, stream);
}

}  // namespace atom
