/*
 * atom.h -- C ABI of libatom, the Atom copy/reduce datapath for AMD MI355X
 * (gfx950).
 *
 * Source of the semantics: "Purlin: Separating Orchestration from the
 * Datapath of Collectives" (arXiv 2609.36954).
 *  - Abstract: a collective is defined by its input layout, its output
 *    layout and one operation (copy or reduce); the Atom datapath supplies
 *    those two primitives; SNAC (Stage, Notify, And Consume) derives the
 *    coordination from the layouts.
 *  - Figure 4: ReduceScatter combines partition k of every input into y_k at
 *    rank k; AllGather places every y_k in rank order at every rank;
 *    AllToAll gives rank j partition j of every source.
 *  - Figure 6: AllReduce composed from ReduceScatter and AllGather, chunk by
 *    chunk.
 *  - Table 2: the variable-length (V) variants.
 *  - Table 3: chunk size = bandwidth-delay product rounded to the closest
 *    power of two.
 *
 * Here the P "ranks" are P buffers in one GPU's memory. The reduction is a
 * sum accumulated in binary32 in rank order 0..P-1 and rounded once to the
 * element type (round to nearest, ties to even).
 *
 * General conventions (every entry point)
 *  - Device pointers are plain HIP device addresses (hipMalloc / torch CUDA
 *    tensors) on the current HIP device. Host arrays (pointer lists, counts)
 *    are read during the call and copied; the caller may free them on return.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls are
 *    asynchronous and stream-ordered; device buffers must stay alive until
 *    the stream has executed the call.
 *  - Every argument is validated on the host before any HIP call, so invalid
 *    arguments return ATOM_ERR_INVALID_ARG / ATOM_ERR_UNSUPPORTED without
 *    touching the GPU. No entry point aborts or throws.
 *  - Zero-sized work returns ATOM_OK without launching anything.
 *  - Out of place only: an output byte range that overlaps any input range
 *    or another output range is ATOM_ERR_INVALID_ARG.
 *  - Any element-aligned pointer is accepted, by every entry point. 16-byte
 *    aligned buffers whose partitions keep 16-byte alignment take the
 *    128-bit vector path; others take an element-wise path with the same
 *    results. Zero-staging calls stay vectorized when the streams sit at a
 *    common offset from 16-byte alignment (element-wise edges), and also
 *    when a part's sources and its destinations sit at different offsets
 *    (each 16-byte store assembled from two source vectors), as long as the
 *    sources of one part (reduce) or the destinations of one segment
 *    (fan-out) agree; staged calls choose per segment, a segment being the
 *    bytes one source sends to one or every destination (vectors when all
 *    its streams share one offset from 16-byte alignment, with element-wise
 *    ends; staged as vectors and consumed by the shifted path when its
 *    sources share one offset and a destination sits at another;
 *    element-wise when its sources disagree); the MoE movement chooses per
 *    call.
 *  - Calls that use the per-device workspace (the SNAC staging ring and its
 *    flags) are ordered by their stream; two such calls on different streams
 *    of one device must not overlap in time.
 *  - HIP graph capture: every call only launches kernels on `stream` (no
 *    memset, no host synchronization), so calls can be captured and
 *    replayed. The workspace is allocated on a device's first staged call
 *    and grows when a call needs a larger ring; a staged call that would
 *    have to allocate while `stream` is being captured returns
 *    ATOM_ERR_UNSUPPORTED and enqueues nothing, so make one eager call of
 *    the largest staged configuration first. The workspace only grows, and
 *    replaced rings stay allocated until the process ends, so a captured
 *    graph stays valid after later calls.
 */
#ifndef ATOM_H
#define ATOM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATOM_MAX_RANKS 16

typedef enum atom_status {
    ATOM_OK = 0,
    ATOM_ERR_INVALID_ARG = 1,  /* malformed arguments, overlap, misalignment   */
    ATOM_ERR_UNSUPPORTED = 2,  /* a layout/op pair that names no collective    */
    ATOM_ERR_HIP = 3,          /* a HIP runtime call or a launch failed         */
    ATOM_ERR_TIMEOUT = 4,      /* a SNAC wait exceeded its bound on the device  */
    ATOM_ERR_NOMEM = 5,        /* the workspace could not be allocated          */
    ATOM_ERR_LIMIT = 6         /* a staged call does not fit the fixed workspace
                                  of atom_collective_noalloc                    */
} atom_status;

/* The input enums below carry range sentinels so that any 32-bit value a
 * caller passes is a valid value of the type (and is rejected by
 * validation) rather than undefined behaviour in the C++ implementation. */

typedef enum atom_dtype {
    ATOM_DT_BF16 = 0,          /* 2-byte bfloat16 */
    ATOM_DT_F32 = 1,           /* 4-byte IEEE binary32 */
    ATOM_DT_ENUM_MIN = INT32_MIN,
    ATOM_DT_ENUM_MAX = INT32_MAX
} atom_dtype;

typedef enum atom_op {
    ATOM_OP_COPY = 0,          /* move bits unchanged */
    ATOM_OP_SUM = 1,           /* binary32 sum in rank order, rounded once */
    ATOM_OP_ENUM_MIN = INT32_MIN,
    ATOM_OP_ENUM_MAX = INT32_MAX
} atom_op;

/* How P buffers name a layout (Figure 4). n = part_elems (uniform case).
 * PARTITIONED: buffer r holds P partitions of n elements, partition k at
 *              element k*n. V form: buffer r holds P row segments, segment j
 *              = counts[r*P+j] rows of row_elems elements, in j order.
 * SHARD:       buffer k holds the single partition k (n elements).
 * GATHERED:    every buffer holds all P partitions in rank order (P*n).
 * TRANSPOSED:  buffer j holds partition j of every source, in source order
 *              (P*n). V form: sum_r counts[r*P+j] rows, segment of source r
 *              first for smaller r. */
typedef enum atom_layout_kind {
    ATOM_LAYOUT_PARTITIONED = 0,
    ATOM_LAYOUT_SHARD = 1,
    ATOM_LAYOUT_GATHERED = 2,
    ATOM_LAYOUT_TRANSPOSED = 3,
    ATOM_LAYOUT_ENUM_MIN = INT32_MIN,
    ATOM_LAYOUT_ENUM_MAX = INT32_MAX
} atom_layout_kind;

typedef struct atom_layout {
    atom_layout_kind kind;
    int32_t nranks;            /* P, 1..ATOM_MAX_RANKS; must match across in/out */
    void* const* bufs;         /* P device pointers (host array), caller-owned */
    int64_t part_elems;        /* n, uniform case; ignored when counts != NULL */
    const int64_t* counts;     /* NULL, or the V-variant counts (host array):
                                  AllToAllV: P*P row-major, counts[r*P+j] rows
                                  from source r to destination j;
                                  ReduceScatterV / AllGatherV: P entries,
                                  counts[k] rows in partition k. */
    int64_t row_elems;         /* elements per row for counts (>= 1) */
    atom_dtype dtype;          /* must match across in/out */
} atom_layout;

/* Execution options; NULL means defaults. Zero fields take defaults too. */
#define ATOM_F_STAGED 0x1u     /* run through SNAC with a staging ring */
#define ATOM_F_NO_NT  0x2u     /* use ordinary (cached) stores for every output.
                                 Default: streaming (non-temporal) stores,
                                 except for zero-staging messages under
                                 1 MiB, whose outputs are kept in the caches
                                 for the operation that reads them next */
#define ATOM_F_XCD_ORDER 0x4u /* zero-staging kernels give each XCD one
                                 contiguous range of tiles (default: plain
                                 workgroup order; measured within noise) */
#define ATOM_F_COUNTED 0x8u   /* staged calls: always notify through the
                                 ring slots' count words. Default: a staged
                                 call whose ring holds every chunk (each
                                 staged once), each of whose segments has
                                 its sources and destinations at one offset
                                 from 16-byte alignment, which stages at most
                                 16 MiB and sets no num_wgs carries its
                                 notify in the staged
                                 data itself: each staged 4-byte word is
                                 written next to a tag holding the call's
                                 sequence number, by one 64-bit store, and
                                 the consumer waits for its words' tags
                                 (atom_plan_info.snac_tagged). Same results;
                                 ignored by zero-staging calls. */
typedef struct atom_config {
    int64_t chunk_bytes;       /* SNAC chunk (notify unit); power of two in
                                  [64 KiB, 16 MiB]; default: a copying stage
                                  (AllGather(V), AllToAll(V)) 512 KiB, 2 MiB
                                  when its largest segment is at least
                                  256 MiB; a reducing one 2 MiB. A partition
                                  smaller than the chunk is staged as one
                                  chunk of whole pieces (plan_query reports
                                  the chunk used). */
    int32_t stages;            /* 16-byte vectors in flight per lane: 1, 2, 4 or 8
                                  (0: chosen per collective) */
    int32_t num_wgs;           /* workgroups to launch; 0 = derived from size */
    uint32_t flags;            /* ATOM_F_* */
    int32_t ring_slots;        /* SNAC ring depth D: 1..64; default: enough
                                  slots for 32 MiB in flight (at least 4) */
    int32_t piece_bytes;       /* SNAC task granule: a power of two in
                                  [16 KiB, chunk]; 0: default */
    int32_t wait_us;           /* bound of one SNAC wait in microseconds; 0:
                                  1 s. On expiry the kernel records a timeout
                                  (see atom_sync_status), drops the waiting
                                  task and drains; the output is incomplete. */
    int32_t lanes;             /* threads per workgroup: 64, 128 or 256, and
                                  for staged calls also 512 (a wider
                                  zero-staging request is
                                  ATOM_ERR_UNSUPPORTED); 0: chosen per
                                  collective and size (staged: 512) */
    int32_t jitter_us;         /* test hook of the staged path, 0..10000 (0:
                                  off): before each notify and each consume,
                                  the task's workgroup waits a pseudo-random
                                  0..jitter_us microseconds drawn from
                                  (jitter_seed, task), so that hand-offs run
                                  at other than their natural timing. The
                                  result is unchanged; only time is added. */
    uint32_t jitter_seed;
    int32_t snac_lead;         /* SNAC ticket order: chunks staged ahead of
                                  the first consumer, 0..64, clamped to the
                                  ring depth (0: half the ring depth). Smaller
                                  leads leave slack
                                  slots so a producer seldom waits for a
                                  slot to be freed. */
    uint64_t* trace;           /* measurement hook of the staged path (NULL:
                                  off): a device array, caller-owned, of at
                                  least 4 * atom_plan_info.snac_tasks
                                  entries. Task t (its ticket) writes entry
                                  4t: the device clock when its workgroup
                                  took the ticket; 4t+1: when its wait
                                  ended; 4t+2: when its work (stage, or
                                  consume) had completed; 4t+3: its
                                  workgroup index | producer flag << 32 |
                                  wait given up << 33. The clock is the
                                  device's constant-rate counter
                                  (hipDeviceAttributeWallClockRate kHz).
                                  Results are unchanged. */
} atom_config;

/* The collective that a pair of layouts and an op names (Figure 4/6,
 * Table 2). */
typedef enum atom_collective_kind {
    ATOM_COLL_NONE = 0,
    ATOM_COLL_REDUCE_SCATTER = 1,     /* PARTITIONED -> SHARD,      SUM  */
    ATOM_COLL_ALL_GATHER = 2,         /* SHARD       -> GATHERED,   COPY */
    ATOM_COLL_ALL_TO_ALL = 3,         /* PARTITIONED -> TRANSPOSED, COPY */
    ATOM_COLL_ALL_TO_ALL_V = 4,       /* same, with P*P counts           */
    ATOM_COLL_ALL_REDUCE = 5,         /* PARTITIONED -> GATHERED,   SUM  */
    ATOM_COLL_REDUCE_SCATTER_V = 6,   /* RS with P partition counts      */
    ATOM_COLL_ALL_GATHER_V = 7        /* AG with P partition counts      */
} atom_collective_kind;

/* What the planner derived, for inspection without a GPU. */
typedef struct atom_plan_info {
    atom_collective_kind kind;
    int32_t nranks;
    int32_t staged;            /* 1 when the call would run through SNAC */
    int32_t vector_path;       /* 1: the 128-bit vector path (every stream
                                  16-byte aligned, at one common offset from
                                  it, or shifted, see below); 0: element-wise */
    int64_t elems_per_rank_in; /* elements of each input buffer */
    int64_t elems_per_rank_out[ATOM_MAX_RANKS];  /* elements of each output */
    int64_t credited_bytes;    /* algorithmic bytes: each input element read
                                  once, each output element written once */
    int64_t chunk_bytes;       /* SNAC chunk, when staged */
    int64_t num_chunks;        /* SNAC chunks, when staged */
    int32_t ring_slots;
    int32_t num_wgs;           /* workgroups the launch would use (all rows) */
    int32_t lanes;             /* threads per workgroup */
    int32_t stages;            /* 16-byte slots per lane per tile (staged:
                                  in flight while fanning out) */
    int32_t streaming_stores;  /* 1: outputs written with non-temporal
                                  stores; 0: ordinary stores */
    int32_t grid_rows;         /* 1, or the parts of a small uniform reduce
                                  launched as a tiles x parts grid */
    int32_t shifted;           /* 1 when the vector path moves some part or
                                  segment between a source and a destination
                                  at different offsets from 16-byte alignment
                                  (each 16-byte store assembled from two
                                  neighbouring source vectors) */
    int32_t snac_lead;         /* SNAC: chunks staged ahead of the consumers */
    int64_t snac_tasks;        /* SNAC: stage + consume tasks (2 * chunks *
                                  pieces per chunk); 0 when not staged */
    int32_t snac_tagged;       /* SNAC: 1 when the call hands off through
                                  tagged words (see ATOM_F_COUNTED), 0 through
                                  the slot count words */
    int32_t reserved;
} atom_plan_info;

/* Atom copy (abstract: the copy primitive). Copies `bytes` bytes from src to
 * dst on `stream`. Both are device pointers; the ranges must not overlap.
 * Returns ATOM_OK, ATOM_ERR_INVALID_ARG (NULL with bytes > 0, overlap) or
 * ATOM_ERR_HIP. */
atom_status atom_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Atom reduce (abstract: the reduction primitive). dst[i] = sum over r of
 * srcs[r][i], i < count, in binary32, rank order, one rounding to dtype.
 * srcs is a host array of nsrcs (1..ATOM_MAX_RANKS) device pointers; dst
 * must not overlap any source. op must be ATOM_OP_SUM (ATOM_OP_COPY with
 * nsrcs == 1 is a copy). Returns ATOM_OK, ATOM_ERR_INVALID_ARG,
 * ATOM_ERR_UNSUPPORTED or ATOM_ERR_HIP. */
atom_status atom_reduce(void* dst, const void* const* srcs, int32_t nsrcs,
                        int64_t count, atom_dtype dtype, atom_op op,
                        void* stream);

/* A collective named by its layouts and op (abstract; Figures 4 and 6;
 * Table 2). The pair (in->kind, out->kind, op) selects the collective as
 * listed at atom_collective_kind; other pairs return ATOM_ERR_UNSUPPORTED.
 * Both layouts must agree on nranks, dtype and (V forms) counts/row_elems;
 * out->counts may be NULL. With cfg->flags & ATOM_F_STAGED every collective
 * runs through SNAC (abstract; Figure 6; Figure 16 for the V forms on
 * ordinary buffers): its layouts become a list of segments (the bytes one
 * source sends to one or every destination), chunks of cfg->chunk_bytes of
 * each are staged (copied, or reduced in rank order) in a ring of
 * cfg->ring_slots slots, notified through device-memory flags (a call that
 * stages each chunk once: through a tag stored with each staged word, see
 * ATOM_F_COUNTED) and
 * consumed by other workgroups; the result equals the zero-staging one bit
 * for bit.
 * Returns ATOM_OK, ATOM_ERR_INVALID_ARG, ATOM_ERR_UNSUPPORTED,
 * ATOM_ERR_NOMEM or ATOM_ERR_HIP. A SNAC wait that runs out on the device is
 * reported by atom_sync_status, not here (the call returns before the
 * kernel runs); only the call whose wait ran out is incomplete. */
atom_status atom_collective(const atom_layout* in, const atom_layout* out,
                            atom_op op, const atom_config* cfg, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * collective as atom_collective, but a staged call takes its ring and flags
 * from a fixed array inside the library (ATOM_NOALLOC_RING_BYTES of ring, and
 * 32 MiB for the tagged words, per device, held from the
 * library's load until the process ends) instead of
 * the growing workspace, so no call allocates. Without cfg->ring_slots the
 * ring depth is cut to what fits; a call whose chunk (as planned: a message
 * smaller than the chunk is staged in a smaller one), or whose chunk times
 * cfg->ring_slots, exceeds ATOM_NOALLOC_RING_BYTES returns ATOM_ERR_LIMIT
 * before anything is launched. Zero-staging calls use no workspace and behave exactly as in
 * atom_collective. Every staged call on one device shares that device's
 * array: two such calls that overlap in time (different streams) race and
 * give wrong results. The first call on a device also enqueues one small
 * kernel that clears the array's flags. Same return codes as
 * atom_collective, plus ATOM_ERR_LIMIT. */
#define ATOM_NOALLOC_RING_BYTES (16 << 20)
atom_status atom_collective_noalloc(const atom_layout* in, const atom_layout* out,
                                    atom_op op, const atom_config* cfg, void* stream);

/* Validation and planning only, no HIP call: fills *info with what
 * atom_collective would do. Same return codes as its validation step. */
atom_status atom_plan_query(const atom_layout* in, const atom_layout* out,
                            atom_op op, const atom_config* cfg,
                            atom_plan_info* info);

/* Synchronizes `stream`, then reads and clears this device's SNAC error
 * words (of the workspace and of the fixed array of
 * atom_collective_noalloc): ATOM_ERR_TIMEOUT if a wait timed out since the
 * last check, else ATOM_OK (ATOM_ERR_HIP if the synchronization fails). A
 * timeout leaves incomplete output in the call it happened in only; calls
 * after it wait normally. (A HIP graph replays one captured call with one
 * sequence number: after a timeout in a replay, the later replays of that
 * same captured call give up their waits too until this check clears the
 * word.) */
atom_status atom_sync_status(void* stream);

/* Table 3: bandwidth-delay product R*tau in bytes rounded to the closest
 * power of two (ties go to the larger). Returns 0 for non-positive input. */
int64_t atom_bdp_chunk_bytes(double bytes_per_s, double round_trip_s);

/* A static, human-readable name for a status code. */
const char* atom_status_string(atom_status s);

/* The HIP runtime's description of the error behind this thread's last
 * ATOM_ERR_HIP (a static string; "no HIP error" if there was none). */
const char* atom_last_error(void);

/* ---- Expert-parallel MoE dispatch and combine ---------------------------
 * Table 2 lists expert parallelism among the uses of AllToAll(V): tokens are
 * dispatched to experts and the expert outputs combined. P ranks host E
 * experts (E a multiple of P): rank j hosts experts [j*E/P, (j+1)*E/P).
 * Every rank holds T tokens; token t of rank r picks k experts, the ids
 * expert_ids[r][t*k + c] for choice c = 0..k-1 (entry i = t*k + c). An id
 * outside [0, E) routes nowhere.
 *
 * Dispatch is the AllToAllV whose destinations are the experts: expert e
 * receives one row per entry routed to it, from every source rank in rank
 * order and, within a source, in entry order; rank j's dispatch buffer holds
 * its experts' rows back to back in expert order (each expert's rows are
 * contiguous, ready for a grouped expert computation). Combine is its way
 * back: out[r][t] = sum over c of weights[r][t*k + c] * (the row entry
 * t*k + c was dispatched to), accumulated in binary32 from +0 by one fused
 * multiply-add per choice in choice order, rounded once to the row dtype.
 *
 * All arrays named below are device memory owned by the caller. Calls are
 * stream-ordered and asynchronous; arguments are validated on the host
 * before anything is launched. Buffers may not overlap unless stated. */

#define ATOM_MOE_MAX_EXPERTS 1024
#define ATOM_MOE_MAX_TOPK 16
#define ATOM_MOE_MAX_ENTRIES (1 << 20)   /* T*k per rank */

typedef struct atom_moe_routing {
    int32_t nranks;                    /* P, 1..ATOM_MAX_RANKS */
    int32_t num_experts;               /* E, a multiple of P, at most
                                          ATOM_MOE_MAX_EXPERTS */
    int32_t topk;                      /* k, 1..ATOM_MOE_MAX_TOPK */
    int32_t reserved;                  /* must be 0 */
    int64_t tokens;                    /* T per rank, T*k <= ATOM_MOE_MAX_ENTRIES */
    const int32_t* const* expert_ids;  /* host array of P device pointers, each
                                          T*k int32 (token-major); read only */
    int32_t* const* positions;         /* host array of P device pointers, each
                                          T*k int32; written by atom_moe_route:
                                          the row of entry i in the dispatch
                                          buffer of the rank hosting its expert,
                                          -1 for an invalid id */
    int32_t* counts;                   /* P*E int32, written by atom_moe_route:
                                          counts[r*E + e] = rows rank r sends
                                          to expert e */
    int64_t* recv_rows;                /* P int64, written by atom_moe_route:
                                          rows rank j receives */
    void* scratch;                     /* atom_moe_scratch_bytes(...) bytes,
                                          16-byte aligned, used by
                                          atom_moe_route only */
} atom_moe_routing;

/* Bytes of scratch atom_moe_route needs for this shape (0 for invalid
 * arguments). */
int64_t atom_moe_scratch_bytes(int32_t nranks, int32_t num_experts,
                               int32_t topk, int64_t tokens);

/* Routing: fills positions, counts and recv_rows from expert_ids (the
 * layout of the dispatch). Returns ATOM_OK, ATOM_ERR_INVALID_ARG (a field
 * out of range, a NULL pointer, misaligned scratch) or ATOM_ERR_HIP. */
atom_status atom_moe_route(const atom_moe_routing* rt, void* stream);

/* Dispatch: for every entry with a valid id whose position is below
 * capacity_rows, copies row t of x[r] (row_elems elements of dtype) to row
 * positions[r][i] of out[j], j the rank hosting the entry's expert. Each
 * token row is read once and written once per choice. x: host array of P
 * device pointers to T rows; out: host array of P device pointers to
 * capacity_rows rows each (rows no entry lands on are not written). Uses
 * the positions of the last atom_moe_route on rt. Rows at or beyond
 * capacity_rows are dropped; recv_rows tells how many would land. Any
 * element-aligned buffers are accepted: 16-byte aligned buffers with rows
 * of a 16-byte multiple take the 128-bit kernels, others an element-wise
 * kernel (one tile per token row, ordinary stores) with the same results.
 * cfg may be NULL (defaults); of its fields lanes (64, 128, 256), stages
 * (16-byte slots per lane per tile; ignored by the element-wise kernel),
 * num_wgs and ATOM_F_NO_NT apply, the SNAC fields are ignored, and
 * ATOM_F_STAGED or ATOM_F_XCD_ORDER is ATOM_ERR_UNSUPPORTED. Returns
 * ATOM_OK, ATOM_ERR_INVALID_ARG, ATOM_ERR_UNSUPPORTED or ATOM_ERR_HIP. */
atom_status atom_moe_dispatch(const atom_moe_routing* rt, const void* const* x,
                              void* const* out, int64_t capacity_rows,
                              int64_t row_elems, atom_dtype dtype,
                              const atom_config* cfg, void* stream);

/* Combine: out[r] row t = round(sum over c of weights[r][t*k + c] * y row),
 * the y row being row positions[r][i] of y[j] for the entry's rank j;
 * entries with an invalid id or a position at or beyond capacity_rows are
 * skipped. y: host array of P device pointers to capacity_rows rows (the
 * expert outputs, in dispatch layout); weights: host array of P device
 * pointers to T*k float; out: host array of P device pointers to T rows.
 * Same alignment rule, cfg fields and return codes as atom_moe_dispatch. */
atom_status atom_moe_combine(const atom_moe_routing* rt, const void* const* y,
                             const float* const* weights, void* const* out,
                             int64_t capacity_rows, int64_t row_elems,
                             atom_dtype dtype, const atom_config* cfg, void* stream);

/* Rate of the device clock that atom_config.trace stamps count, in kHz,
 * for the current HIP device. Returns ATOM_OK, ATOM_ERR_INVALID_ARG (khz
 * NULL) or ATOM_ERR_HIP. */
atom_status atom_device_clock_khz(int32_t* khz);

/* Library version, (major << 16) | minor. */
int32_t atom_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATOM_H */
