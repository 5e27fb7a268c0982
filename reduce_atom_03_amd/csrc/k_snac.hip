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
//           into a slot of the staging ring;
//   Notify  after its stores are released at agent scope it adds 1 to the
//           slot's `ready` counter;
//   Consume a consumer workgroup acquires `ready` == all pieces of the chunk,
//           copies one piece from the slot to every output (AllGather
//           fan-out) and adds 1 to the slot's `freed` counter, which the
//           producer of the chunk D places later waits for before reuse.
//
// Tasks are claimed from one atomic ticket in an order where every task
// depends only on tasks with smaller tickets: producers of chunks 0..D-1,
// then for each later chunk q the consumers of chunk q-D followed by the
// producers of chunk q, then the consumers of the last D chunks. A claimed
// ticket belongs to a running workgroup, so the lowest unfinished task can
// always proceed: no deadlock for any grid size or occupancy. Every wait is
// bounded; on expiry the error word is set, the task is dropped, and later
// waits give up at once, so the grid always drains.
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

// Lane 0 waits until *flag >= target (bounded), then every wave acquires.
// Returns false when the wait gave up (timeout here or elsewhere).
__device__ __forceinline__ bool wait_at_least(const SnacArgs& a, const unsigned long long* flag,
                                              unsigned long long target, int* s_ok)
{
    if (threadIdx.x == 0) {
        int ok = 1;
        int64_t it = 0;
        while (flag_load_relaxed(flag) < target) {
            if (__hip_atomic_load(a.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
                ++it > a.spin_limit) {
                __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        *s_ok = ok;
    }
    __syncthreads();
    const bool ok = *s_ok != 0;
    if (ok)
        fence_acquire_agent();
    return ok;
}

// Copies `bytes` bytes (a multiple of 16) from src to dst (ndst == 1) or to
// a.dst[q] + dst_off for every q < ndst (fan-out: one load, ndst stores).
template <int U>
__device__ __forceinline__ void copy_piece(const SnacArgs& a, const char* src, char* dst, int ndst,
                                           int64_t dst_off, int64_t bytes, bool nt)
{
    const int lane = threadIdx.x;
    const int nthr = blockDim.x;
    const int64_t step = static_cast<int64_t>(nthr) * U * kVecBytes;
    for (int64_t b0 = 0; b0 < bytes; b0 += step) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t o = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
            if (o < bytes)
                x[u] = ld16(src + o);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t o = b0 + static_cast<int64_t>(u * nthr + lane) * kVecBytes;
            if (o < bytes) {
                if (dst) {
                    st16(dst + o, x[u], nt);
                } else {
                    for (int q = 0; q < ndst; ++q)
                        st16(static_cast<char*>(a.dst[q]) + dst_off + o, x[u], nt);
                }
            }
        }
    }
}

template <int U>
__global__ __launch_bounds__(256) void k_snac_allgather(const SnacArgs a)
{
    __shared__ unsigned int s_ticket;
    __shared__ int s_ok;
    const int64_t S = a.part_bytes;
    const int64_t C = a.chunk_bytes;
    for (;;) {
        if (threadIdx.x == 0)
            s_ticket = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int64_t t = s_ticket;
        __syncthreads();
        if (t >= a.ntasks)
            break;
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
        if (task.produce) {
            // Stage: the slot's previous chunk must be fully consumed.
            if (!wait_at_least(a, a.freed + slot, static_cast<unsigned long long>(use) * a.pieces, &s_ok))
                continue;
            copy_piece<U>(a, static_cast<const char*>(a.src[k]) + cbeg + pbeg, slotp + pbeg, 1, 0, plen,
                          false);
            // Notify: release this wave's stores at agent scope, then count the piece.
            fence_release_agent();
            __syncthreads();
            if (threadIdx.x == 0)
                flag_add_release(a.ready + slot, 1ull);
        } else {
            // Consume: the whole chunk must be staged.
            if (!wait_at_least(a, a.ready + slot, static_cast<unsigned long long>(use + 1) * a.pieces, &s_ok))
                continue;
            copy_piece<U>(a, slotp + pbeg, nullptr, a.P, static_cast<int64_t>(k) * S + cbeg + pbeg, plen,
                          a.nt_store != 0);
            __syncthreads();   // every lane's slot reads have returned (their data was stored)
            if (threadIdx.x == 0)
                flag_add_release(a.freed + slot, 1ull);
        }
    }
}

// Clears the ticket and the slot counters before a SNAC launch (the error
// word is kept until the host reads it). A kernel, not a memset, so the
// sequence can be captured into a graph.
__global__ void k_snac_reset(unsigned long long* ready, unsigned long long* freed, unsigned int* ticket,
                             int slots)
{
    const int i = threadIdx.x;
    if (i < slots) {
        ready[i] = 0;
        freed[i] = 0;
    }
    if (i == 0)
        *ticket = 0;
}

}  // namespace

hipError_t launch_snac_ag(const Plan& p, const Workspace& ws, hipStream_t stream)
{
    if (p.exec != EX_SNAC_AG || !ws.ring || ws.ring_bytes < p.ring_bytes || p.grid < 1 ||
        p.sa.slots < 1 || p.sa.slots > kMaxSlots || p.sa.pieces < 1)
        return hipErrorInvalidValue;
    SnacArgs a = p.sa;
    a.ring = ws.ring;
    a.ready = ws.ready;
    a.freed = ws.freed;
    a.ticket = ws.ticket;
    a.error = ws.error;
    k_snac_reset<<<1, 64, 0, stream>>>(ws.ready, ws.freed, ws.ticket, a.slots);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    k_snac_allgather<4><<<dim3(static_cast<unsigned>(p.grid)), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace atom
