// kargs.hpp -- kernel argument blocks, shared by the host planner and the
// kernels. Plain data only (no HIP types): the planner fills them on the
// host, the launchers pass them by value, so a launch needs no device-side
// descriptor upload. Each block stays well under 4 KiB of kernel arguments.
#pragma once

#include <stdint.h>

// Helpers below are used by the host planner and by the kernels.
#if defined(__HIPCC__) || defined(__HIP__)
#define ATOM_HD __host__ __device__
#else
#define ATOM_HD
#endif

namespace atom {

constexpr int kMaxRanks = 16;
constexpr int kMaxSegs = kMaxRanks * kMaxRanks;
constexpr int kVecBytes = 16;          // one global_load/store_dwordx4
constexpr int kFlagStride = 32;        // SNAC counters sit 256 bytes apart (u64 units)

enum DType : int32_t { DT_BF16 = 0, DT_F32 = 1 };

// Reduce family: dst = sum over nsrc sources, element-wise, in rank order.
// Part k covers source elements [part_off[k], part_off[k+1]).
//  SCATTER: part k is written to dst[k] + (i - part_off[k])   (ReduceScatter(V),
//           and the flat reduce with one part)
//  FANOUT:  part k is written to dst[q] + i for every q < ndst (AllReduce)
enum ReduceMode : int32_t { RM_SCATTER = 0, RM_FANOUT = 1 };

struct ReduceArgs {
    const void* src[kMaxRanks];
    void* dst[kMaxRanks];
    int64_t part_off[kMaxRanks + 1];   // elements
    int64_t tile_begin[kMaxRanks + 1]; // first tile of each part; [nparts] = ntiles
    int64_t ntiles;
    int32_t shift[kMaxRanks];          // per part: slots before its first slot in
                                       // its first tile (tiles start at addresses
                                       // aligned to the tile size in source 0)
    int32_t head[kMaxRanks];           // vector path, per part: elements before its
                                       // first 16-byte boundary (every stream of
                                       // the part is off alignment by the same
                                       // amount); reduced element by element
    int32_t nsrc;
    int32_t ndst;
    int32_t nparts;
    int32_t mode;
    int32_t nt_store;                  // 1: non-temporal output stores
    int32_t xcd_remap;                 // 1: XCD-contiguous tile order
    int32_t grid_parts;                // 0: one-dimensional grid, each tile finds
                                       // its part in tile_begin. Else (small
                                       // messages) the uniform form: nparts parts
                                       // of part_off[1] elements each (part k at
                                       // k * part_off[1]), no heads, one shift
                                       // (shift[0]) and gridDim.x tiles per part;
                                       // part = blockIdx.y
    int32_t shifted;                   // 1: a part's sources sit at one offset from
                                       // 16-byte alignment and its destination(s)
                                       // at another: k_reduce_shift, tiles over the
                                       // part's source vectors plus one
};

// Copy family. Segments are derived in the kernel from row counts:
//  CK_FANOUT:  segment k < nseg_src is source src[k], cnt[k] rows, written
//              to every dst[q] (q < ndst) at byte offset sum_{k'<k} cnt[k']
//              * row_bytes (AllGather(V); atom_copy is one segment).
//  CK_EXCHANGE: segment s = r*P + j moves cnt[s] rows from src[r] (after
//              source r's rows for every j' < j) to dst[j] (after every
//              source r' < r's rows for j)  (AllToAll(V)).
enum CopyKind : int32_t { CK_FANOUT = 0, CK_EXCHANGE = 1 };

struct CopyArgs {
    const void* src[kMaxRanks];
    void* dst[kMaxRanks];
    int64_t row_bytes;
    int64_t ntiles;
    int64_t tile_bytes;                // bytes per tile (multiple of 16)
    int32_t kind;
    int32_t P;                         // ranks (segments: P or P*P)
    int32_t nseg;
    int32_t ndst;                      // fan-out count (CK_FANOUT)
    int32_t esize;                     // element bytes for the element-wise path
    int32_t nt_store;
    int32_t xcd_remap;                 // 1: XCD-contiguous tile order
    int32_t align;                     // 1: tiles start at addresses aligned to
                                       // tile_bytes in the destination (see
                                       // seg_tile_shift)
    int32_t grid_segs;                 // 0: one-dimensional grid, each tile finds
                                       // its segment in seg_tile_begin. Else (small
                                       // messages) the uniform form: grid_segs
                                       // segments of cnt[0] rows, no heads, the same
                                       // tile count each; segment = blockIdx.y, tile
                                       // within it = blockIdx.x
    int32_t block_shift;               // CK_FANOUT blocked order (k_copy_fan_blocked):
                                       // log2 of the tiles per block (a power of
                                       // two, at least the 8 XCDs); -1: every tile
                                       // stores to all outputs
    int32_t shifted;                   // 1: some segment's source and destination
                                       // sit at different offsets from 16-byte
                                       // alignment (each segment's destinations at
                                       // the same one): k_copy_shift, tiles over
                                       // the segment's source vectors plus one
    int64_t nwork;                     // blocked order: workgroup tasks,
                                       // blocks * 2^block_shift * ndst
    int64_t seg_off[kMaxRanks + 1];    // CK_FANOUT: byte offset of segment s in
                                       // the outputs (seg_off[nseg] = their size)
    int32_t cnt[kMaxSegs];             // rows per segment
    int32_t seg_tile_begin[kMaxSegs + 1];
    uint8_t head[kMaxSegs];            // vector path, per segment: bytes before its
                                       // first 16-byte boundary (source and every
                                       // destination off alignment by the same
                                       // amount); copied element by element
};

// SNAC: every collective staged through a ring. The work is a list of
// segments, each a contiguous byte range staged chunk by chunk:
//  SK_GATHER   segment k = source src[k] (cnt[k] rows), written to every
//              dst[q] at byte offset sum_{k'<k} cnt[k'] * row_bytes
//              (AllGather(V); stage = copy)
//  SK_EXCHANGE segment s = r*P + j: cnt[s] rows of src[r] (after source r's
//              rows for every j' < j) to dst[j] (after every source r' < r's
//              rows for j)  (AllToAll(V); stage = copy)
//  SK_SCATTER  segment k = rows [sum_{k'<k} cnt[k'], +cnt[k]) of every
//              source, summed in rank order, written to dst[k] from byte 0
//              (ReduceScatter(V); stage = reduce)
//  SK_ALLRED   as SK_SCATTER, written to every dst[q] at the segment's own
//              offset  (the composed AllReduce of Figure 6; stage = reduce)
enum SnacKind : int32_t { SK_GATHER = 0, SK_EXCHANGE = 1, SK_SCATTER = 2, SK_ALLRED = 3 };

// How a segment moves: every stream at one offset d from 16-byte alignment
// (vectors, element-wise ends when d > 0); its sources at one offset and a
// destination at another (staged as SE_VEC, consumed by the shifted path);
// sources at different offsets (element by element).
enum SnacSegPath : uint8_t { SE_VEC = 0, SE_ELEM = 1, SE_SHIFT = 2 };

struct SnacArgs {
    const void* src[kMaxRanks];        // inputs
    void* dst[kMaxRanks];              // outputs
    char* ring;                        // D slots of chunk_bytes
    unsigned long long* tags;          // tagged ring (tagged calls): one
                                       // 64-bit pair per staged 4-byte word, the
                                       // call's seq in the high half; piece i of
                                       // chunk q at pair (q * pieces + i) * tag_place
    unsigned long long* counts;        // per slot (stride kFlagStride), over every
                                       // chunk the slot has held in this call:
                                       // pieces staged (low 32 bits) and pieces
                                       // consumed (high 32 bits)
    unsigned int* ticket;              // task counter
    unsigned int* error;               // sequence number of the last call whose
                                       // wait timed out (0: none since cleared)
    unsigned int* done;                // workgroups finished (the last one
                                       // clears the counters for the next call)
    unsigned long long* trace;         // measurement hook: 4 clock stamps per
                                       // task (NULL: off)
    int64_t row_bytes;                 // bytes per counted row
    int64_t chunk_bytes;
    int64_t slot_bytes;                // ring slot stride: chunk_bytes plus padding
    int64_t piece_bytes;               // chunk_bytes / pieces
    int64_t nchunks;                   // chunks of every segment together
    int64_t tag_place;                 // tagged calls: pairs per piece place, 4 per
                                       // 16-byte vector (a piece's vectors, plus 64
                                       // when a segment sits off 16-byte alignment)
    int64_t ntasks;                    // 2 * nchunks * pieces
    int64_t wait_ticks;                // bound of one wait: microseconds when
                                       // planned, device-clock ticks at launch
    int64_t budget_ticks;              // bound of a workgroup's whole run
    int64_t jitter_ticks;              // test hook: largest pseudo-random delay
                                       // before a notify or a consume (0: none);
                                       // microseconds when planned, ticks at launch
    uint32_t jitter_seed;
    uint32_t seq;                      // this call's sequence number (never 0)
    int32_t kind;                      // SnacKind
    int32_t P;
    int32_t nseg;
    int32_t pieces;                    // G pieces per chunk
    int32_t slots;                     // D
    int32_t lead;                      // E, 1..D: chunks staged ahead of the
                                       // consumers in the ticket order (the
                                       // other D - E slots are slack, so a
                                       // producer seldom waits for a slot)
    int32_t dtype;                     // for the reducing stage
    int32_t nt_store;
    int32_t static_tasks;              // 1: one workgroup per task, task = blockIdx.x
                                       // (small calls); 0: tasks claimed by ticket
    int32_t tagged;                    // 1: a call on the tagged ring (each chunk
                                       // staged once, one workgroup per task,
                                       // every segment on the vector path): the
                                       // notify is the tag of each staged word;
                                       // 0: ring + slot counts
    int32_t interleave;                // 1: every segment has the same number of
                                       // chunks and chunk q belongs to segment
                                       // q % nseg (sources staged side by side);
                                       // 0: segment-major, found in chunk_begin
    int32_t cnt[kMaxSegs];             // rows per segment
    int32_t chunk_begin[kMaxSegs + 1]; // first chunk of each segment (segment-major)
    uint8_t elem[kMaxSegs];            // SnacSegPath of the segment
    uint8_t head[kMaxSegs];            // SE_VEC and SE_SHIFT segments: the offset d
                                       // of its sources from 16-byte alignment
                                       // (0..15); for d > 0 a piece is staged
                                       // 112 + d bytes into its ring place, its
                                       // first 16 - d bytes and its tail element
                                       // by element
};

// Expert-parallel MoE routing (three kernels: rank within chunks, per-rank
// prefix, place). Entries i = t*k + c of rank r are cut into chunks of kMoeChunk.
constexpr int kMoeChunk = 256;         // entries one wave ranks in order
constexpr int kMoeMaxTopk = 16;
constexpr int kMoeSmallLds = 32 << 10;   // LDS bound of the one-workgroup routing
// Entries per rank up to which the one-workgroup routing runs: one wave
// ranks 64 entries per step, so it is serial in the entries. Measured on
// MI355X (8 ranks, 256 experts, back-to-back calls): 7.0-9.4 us up to 256
// entries against 12.7 us for the three kernels, 13.4 vs 12.8 us at 512.
constexpr int64_t kMoeSmallEntries = 256;

struct MoeRouteArgs {
    const int32_t* ids[kMaxRanks];     // T*k expert ids per rank
    int32_t* pos[kMaxRanks];           // T*k positions per rank (output)
    int32_t* counts;                   // [P][E] rows rank r sends to expert e
    int64_t* recv;                     // [P] rows rank j receives
    int32_t* partial;                  // [P][nch][E]: chunk histograms, then
                                       // rows of expert e in the rank's
                                       // earlier chunks
    int64_t n;                         // entries per rank (T*k)
    int32_t nch;                       // chunks per rank (at least 1)
    int32_t groups;                    // placing workgroups per rank (<= nch)
    int32_t P;
    int32_t E;
    int32_t per;                       // experts per rank
};

// MoE dispatch (token rows -> expert buffers) and combine (expert rows ->
// weighted token rows). One tile is one token's row.
struct MoeMoveArgs {
    const char* src[kMaxRanks];        // dispatch: x_r; combine: y_j
    char* dst[kMaxRanks];              // dispatch: out_j; combine: out_r
    const int32_t* ids[kMaxRanks];
    const int32_t* pos[kMaxRanks];
    const float* w[kMaxRanks];         // combine: gate weights, T*k per rank
    int64_t T;                         // tokens per rank
    int64_t cap;                       // rows of each expert-side buffer
    int64_t row_bytes;                 // multiple of 16
    int64_t piece_bytes;               // bytes of a row per tile: lanes * U * 16
    int64_t pieces;                    // tiles per token row
    int64_t ntiles;                    // P * T * pieces
    int32_t P;
    int32_t E;
    int32_t per;
    int32_t k;
    int32_t dtype;
    int32_t nt_store;
    int32_t elem;                      // 1: a buffer or the row size is off 16-byte
                                       // alignment: one tile per token row, moved
                                       // element by element (piece = the row)
};

// Kernel arguments of a launch are limited to 4 KiB.
static_assert(sizeof(ReduceArgs) <= 4096 && sizeof(CopyArgs) <= 4096 && sizeof(SnacArgs) <= 4096 &&
                  sizeof(MoeRouteArgs) <= 4096 && sizeof(MoeMoveArgs) <= 4096,
              "kernel argument block too large");

// Bytes before a segment's first byte in its first tile when tiles are
// aligned to `tile_bytes` at the destination address `dst_addr` (the same
// arithmetic on the host, to count tiles, and on the device, to place them).
// Tiles are lanes x slots x 16 bytes with both factors powers of two, so the
// remainder is a mask (a 64-bit remainder costs a kernel ~100 instructions).
ATOM_HD inline int64_t seg_tile_shift(uint64_t dst_addr, int64_t tile_bytes)
{
    return static_cast<int64_t>(dst_addr & (static_cast<uint64_t>(tile_bytes) - 1));
}

}  // namespace atom
