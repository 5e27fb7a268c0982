/*
 * oracle.h -- plain CPU reference of the Atom copy/reduce collectives.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or helper with the GPU library.
 *
 * Semantics follow "Purlin: Separating Orchestration from the Datapath of
 * Collectives" (arXiv 2609.36954): a collective is defined by an input
 * layout, an output layout and a copy or reduce operation (abstract);
 * Figure 4 gives the ReduceScatter, AllGather and AllToAll layouts;
 * Figure 6 composes AllReduce from ReduceScatter and AllGather; Table 2
 * names the variable-length (V) variants. The reduction is a sum.
 *
 * Conventions
 *  - P virtual ranks, 1 <= P <= 64. Buffers are host arrays.
 *  - dtype: ORC_BF16 (raw uint16 bit patterns) or ORC_F32.
 *  - Partitioned input x_r holds P partitions of n elements: partition k is
 *    x_r[k*n, (k+1)*n).
 *  - A sum is accumulated in binary32 in rank order 0..P-1, starting from the
 *    value of rank 0, and rounded once to the element type (round to nearest,
 *    ties to even). A NaN result becomes the quiet NaN (hi16 | 0x0040).
 *  - Return value: 0 on success, -1 on a bad argument, -2 when out of memory.
 *  - Loops over output elements may run on several OpenMP threads; each
 *    element's own summation order never changes.
 */
#ifndef ORACLE_H
#define ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_BF16 = 0, ORC_F32 = 1 };

/* dst[i] = round_T(f32(s_0[i]) + f32(s_1[i]) + ... + f32(s_{P-1}[i])), m elements. */
int orc_reduce(int P, int64_t m, int dtype, const void* const* srcs, void* dst);

/* ReduceScatter: y_k[i] = sum over r of x_r[k*n + i]; y_k has n elements. */
int orc_reduce_scatter(int P, int64_t n, int dtype, const void* const* x, void* const* y);

/* AllGather: out_j[k*n + i] = z_k[i] for every destination j. */
int orc_all_gather(int P, int64_t n, int64_t esize, const void* const* z, void* const* out);

/* AllToAll: out_j[r*n + i] = x_r[j*n + i]. */
int orc_all_to_all(int P, int64_t n, int64_t esize, const void* const* x, void* const* out);

/* AllToAllV over rows of row_bytes bytes. C is P*P row-major, C[r*P + j] =
 * rows that source r sends to destination j. Source r's rows are grouped by
 * destination in destination order; out_j receives the segments of every
 * source in source order and holds sum_r C[r][j] rows. */
int orc_all_to_all_v(int P, const int64_t* C, int64_t row_bytes,
                     const void* const* x, void* const* out);

/* AllReduce composed as AllGather(ReduceScatter(x)): one rounding to T. */
int orc_all_reduce(int P, int64_t n, int dtype, const void* const* x, void* const* out);

/* ReduceScatterV: partition k has cnt[k] elements on every rank; partitions
 * are packed in k order; y_k[i] = sum over r of x_r[o_k + i], o_k = sum_{k'<k} cnt[k']. */
int orc_reduce_scatter_v(int P, const int64_t* cnt, int dtype,
                         const void* const* x, void* const* y);

/* AllGatherV: out_j[o_k + i] = z_k[i] (in bytes: element size esize). */
int orc_all_gather_v(int P, const int64_t* cnt, int64_t esize,
                     const void* const* z, void* const* out);

/* ---- Expert-parallel MoE dispatch and combine ------------------------
 * Table 2 lists expert parallelism among the uses of AllToAll(V): tokens are
 * dispatched to experts and the expert outputs combined. P ranks host E
 * experts (E a multiple of P), rank j the experts [j*E/P, (j+1)*E/P). Every
 * rank holds T tokens; token t of rank r picks k experts ids_r[t*k + c]
 * (c = 0..k-1), entry i = t*k + c. An id outside [0, E) routes nowhere.
 *
 * Route: the dispatch is an AllToAllV whose destinations are the experts.
 * Expert e receives one row per entry routed to it, from every source rank
 * in rank order and, within a source, in entry order; rank j's buffer holds
 * its experts' rows back to back in expert order. pos_r[i] is the row of
 * entry i in the buffer of the rank hosting its expert (-1 if its id is
 * invalid), counts[r*E + e] the rows r sends to e, recv[j] the rows rank j
 * receives. */
int orc_moe_route(int P, int E, int k, int64_t T, const int32_t* const* ids,
                  int32_t* const* pos, int32_t* counts, int64_t* recv);

/* Dispatch: out_j[pos_r[i]] = row t = i / k of x_r, for every entry with a
 * valid id and pos_r[i] < cap (rows of row_bytes bytes; other rows of out_j
 * are left as they are). */
int orc_moe_dispatch(int P, int E, int k, int64_t T, const int32_t* const* ids,
                     const int32_t* const* pos, int64_t cap, int64_t row_bytes,
                     const void* const* x, void* const* out);

/* Combine: out_r[t][h] = round_T(acc_k), acc_0 = +0, acc_{c+1} =
 * fma_binary32(w_r[t*k + c], y_j[pos_r[t*k + c]][h], acc_c) in choice order
 * c = 0..k-1, where j hosts the entry's expert; entries with an invalid id or
 * pos_r[i] >= cap are skipped. Rows have H elements of dtype. */
int orc_moe_combine(int P, int E, int k, int64_t T, const int32_t* const* ids,
                    const int32_t* const* pos, const float* const* w, int64_t cap,
                    int64_t H, int dtype, const void* const* y, void* const* out);

/* Number of OpenMP threads the loops above use. */
int orc_threads(void);
/* Threads used by later calls (n >= 1); results do not depend on it. */
int orc_set_threads(int n);

#ifdef __cplusplus
}
#endif

#endif /* ORACLE_H */
