// plan.hpp -- host planner: argument validation and derivation of the
// collective, its sizes and its launch from a pair of layouts and an op.
// Pure host C++ (no HIP calls), so every rule here is testable on a CPU.
#pragma once

#include "../../include/atom.h"
#include "kargs.hpp"

namespace atom {

enum Exec : int32_t {
    EX_NONE = 0,      // nothing to launch (zero-sized)
    EX_REDUCE = 1,    // reduce family kernel (ReduceArgs)
    EX_COPY = 2,      // copy family kernel (CopyArgs)
    EX_SNAC_COPY = 3,   // SNAC with a copying stage (SnacArgs: AllGather(V), AllToAll(V))
    EX_SNAC_REDUCE = 4  // SNAC with a reducing stage (SnacArgs: ReduceScatter(V), AllReduce)
};

// The scalar part of a plan. Planning resets only this part (and the
// output sizes); the one argument block a plan uses is filled by its
// builder, so a call never clears the kilobytes of the other blocks.
struct PlanHead {
    atom_collective_kind kind = ATOM_COLL_NONE;
    Exec exec = EX_NONE;
    int32_t dtype = DT_BF16;
    int32_t esize = 2;
    int32_t P = 0;
    int32_t vec = 0;          // 1: 128-bit vector path
    int32_t U = 1;            // 16-byte slots per lane per tile
    int32_t wg = 256;         // threads per workgroup
    int64_t grid = 0;         // workgroups launched
    int64_t credited_bytes = 0;
    int64_t in_elems = 0;
    // SNAC
    int32_t slots = 0;
    int64_t chunk_bytes = 0;
    int64_t ring_bytes = 0;
    int32_t snac_shifted = 0; // 1: some segment is consumed by the shifted path
};

struct Plan : PlanHead {
    int64_t out_elems[kMaxRanks] = {};
    ReduceArgs ra;            // exec == EX_REDUCE
    CopyArgs ca;              // exec == EX_COPY
    SnacArgs sa;              // exec == EX_SNAC_COPY / EX_SNAC_REDUCE

    void reset()
    {
        static_cast<PlanHead&>(*this) = PlanHead();
        for (int64_t& e : out_elems)
            e = 0;
    }
};

// Defaults and limits.
constexpr int64_t kDefaultChunkAllGather = 512 << 10; // staged defaults, measured on MI355X
constexpr int64_t kHugeCopySegment = 256 << 20;      // copying stage: from this largest segment up,
constexpr int64_t kHugeCopyChunk = 2 << 20;          // 2 MiB chunks
constexpr int64_t kDefaultChunkAllReduce = 2 << 20;
constexpr int64_t kMinChunk = 64 << 10;
constexpr int64_t kMaxChunk = 16 << 20;
constexpr int32_t kDefaultSlots = 4;
constexpr int32_t kMaxSlots = 64;
constexpr int64_t kPieceBytes = 64 << 10;            // SNAC task granule, reducing stage
constexpr int64_t kCopyPieceBytes = 32 << 10;        // SNAC task granule, copying stage
constexpr int64_t kMinAutoPiece = 8 << 10;           // smallest granule chosen for small partitions
constexpr int64_t kSnacInflightBytes = 32 << 20;     // default ring: one on-chip BDP
constexpr int64_t kSnacGrid = 512;                   // persistent SNAC workgroups (2 per CU)
constexpr int64_t kSlotPad = 256;                    // bytes past each ring slot's chunk (room for a
                                                     // piece staged 112 + d bytes in, d < 16)
constexpr int64_t kSnacStaticTasks = 256;            // up to this many tasks: one workgroup each, no ticket
constexpr int64_t kTagBytes = 32 << 20;              // tagged ring of staged calls that stage each
                                                     // chunk once (8 bytes per staged 4): 16 MiB of
                                                     // staged data
constexpr int64_t kMaxGrid = 1 << 20;                // a multiple of the XCD count
constexpr int64_t kXcdCount = 8;                     // XCDs of an MI355X; workgroup w runs on XCD w mod 8
constexpr int64_t kFanBlockBytes = 8 << 20;          // blocked fan-out: bytes of source per block
// Blocked fan-out: one workgroup per task up to this grid. A grid stride
// would send each finished workgroup 2^20 tasks ahead, spreading the chip's
// work over many blocks and losing their L2 reuse (measured: 1 GiB
// partitions at 4.1 instead of 5.3 TB/s).
constexpr int64_t kMaxGridBlocked = int64_t(1) << 30;
constexpr int64_t kSmallSlots = 256 * 256;           // below: the latency path
constexpr int64_t kDefaultWaitUs = 1000000;          // one SNAC wait: 1 s
constexpr int64_t kMaxJitterUs = 10000;              // SNAC test hook: largest delay
// Ring of the fixed workspace that atom_collective_noalloc uses.
constexpr int64_t kStaticRingBytes = ATOM_NOALLOC_RING_BYTES;

// MoE routing and movement plans.
struct MoeRoutePlan {
    MoeRouteArgs a;
    int32_t scan_threads = 64;         // prefix workgroup: one thread per expert
    bool small = false;                // one-workgroup routing (one chunk per rank)
};

struct MoeMovePlan {
    MoeMoveArgs a;
    int64_t grid = 0;
    int32_t wg = 64;                   // lanes per workgroup
    int32_t U = 1;                     // 16-byte slots per lane per tile
    int64_t credited_bytes = 0;        // when every id is valid and fits
};

int64_t moe_scratch_bytes(int32_t P, int32_t E, int32_t k, int64_t T);
atom_status plan_moe_route(const atom_moe_routing* rt, MoeRoutePlan* p);
// combine == false: dispatch (src = x, dst = out, w unused);
// combine == true: combine (src = y, dst = out, w = weights).
atom_status plan_moe_move(const atom_moe_routing* rt, bool combine, const void* const* src,
                          const float* const* w, void* const* dst, int64_t cap, int64_t row_elems,
                          atom_dtype dtype, const atom_config* cfg, MoeMovePlan* p);

atom_status plan_copy(void* dst, const void* src, size_t bytes, const atom_config* cfg,
                      Plan* p);
atom_status plan_reduce(void* dst, const void* const* srcs, int32_t nsrcs, int64_t count,
                        atom_dtype dtype, atom_op op, const atom_config* cfg, Plan* p);
atom_status plan_collective(const atom_layout* in, const atom_layout* out, atom_op op,
                            const atom_config* cfg, Plan* p);
// max_ring_bytes > 0: a staged plan must fit a ring of that many bytes (the
// ring depth is cut to fit unless the caller set it; else ATOM_ERR_LIMIT).
atom_status plan_collective_ex(const atom_layout* in, const atom_layout* out, atom_op op,
                               const atom_config* cfg, int64_t max_ring_bytes, Plan* p);
void plan_fill_info(const Plan& p, atom_plan_info* info);
int64_t bdp_chunk_bytes(double bytes_per_s, double round_trip_s);

}  // namespace atom
