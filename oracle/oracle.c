/*
 * oracle.c -- plain CPU reference of the Atom copy/reduce collectives.
 *
 * TEST INFRASTRUCTURE: used only by the tests, the smoke check and the
 * benchmark's CPU-baseline leg. Written as the definitions read, with no
 * blocking, fusion or reordering; see oracle.h for the conventions.
 *
 * Build without fast-math and without contraction so that every binary32
 * addition is one correctly rounded IEEE operation (the MoE combine's fused
 * multiply-add is the explicit C99 fmaf, one rounding by definition):
 *   gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_MAX_P 64

/* ---- element helpers ------------------------------------------------ */

/* bfloat16 is the upper half of a binary32: widening is a 16-bit shift. */
static float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even. Adding 0x7FFF plus
 * the lowest kept bit to the discarded half carries into the kept half
 * exactly when the discarded half is above one half, or equal to one half
 * with an odd kept part. Overflow carries into the exponent and yields inf. */
static uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static float orc_load(const void* base, int dtype, int64_t i)
{
    if (dtype == ORC_BF16)
        return orc_bf16_to_f32(((const uint16_t*)base)[i]);
    return ((const float*)base)[i];
}

static void orc_store(void* base, int dtype, int64_t i, float v)
{
    if (dtype == ORC_BF16)
        ((uint16_t*)base)[i] = orc_f32_to_bf16(v);
    else
        ((float*)base)[i] = v;
}

static int orc_bad_p(int P) { return P < 1 || P > ORC_MAX_P; }
static int orc_bad_dtype(int dtype) { return dtype != ORC_BF16 && dtype != ORC_F32; }
static int64_t orc_esize(int dtype) { return dtype == ORC_BF16 ? 2 : 4; }

/* The sum of element e of P equally shaped arrays, in rank order. */
static float orc_sum_at(int P, int dtype, const void* const* srcs, int64_t e)
{
    float acc = orc_load(srcs[0], dtype, e);
    for (int r = 1; r < P; ++r)
        acc = acc + orc_load(srcs[r], dtype, e);
    return acc;
}

/* ---- reduce --------------------------------------------------------- */

int orc_reduce(int P, int64_t m, int dtype, const void* const* srcs, void* dst)
{
    if (orc_bad_p(P) || orc_bad_dtype(dtype) || m < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        orc_store(dst, dtype, i, orc_sum_at(P, dtype, srcs, i));
    return 0;
}

/* ---- ReduceScatter (Figure 4, top) ---------------------------------- */

int orc_reduce_scatter(int P, int64_t n, int dtype, const void* const* x, void* const* y)
{
    if (orc_bad_p(P) || orc_bad_dtype(dtype) || n < 0)
        return -1;
    for (int k = 0; k < P; ++k) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i)
            orc_store(y[k], dtype, i, orc_sum_at(P, dtype, x, (int64_t)k * n + i));
    }
    return 0;
}

/* ---- AllGather (Figure 4, top) -------------------------------------- */

int orc_all_gather(int P, int64_t n, int64_t esize, const void* const* z, void* const* out)
{
    if (orc_bad_p(P) || n < 0 || esize < 1)
        return -1;
    const int64_t blk = n * esize;
#pragma omp parallel for collapse(2) schedule(static)
    for (int j = 0; j < P; ++j)
        for (int k = 0; k < P; ++k)
            memcpy((char*)out[j] + (int64_t)k * blk, z[k], (size_t)blk);
    return 0;
}

/* ---- AllToAll (Figure 4, bottom) ------------------------------------ */

int orc_all_to_all(int P, int64_t n, int64_t esize, const void* const* x, void* const* out)
{
    if (orc_bad_p(P) || n < 0 || esize < 1)
        return -1;
    const int64_t blk = n * esize;
#pragma omp parallel for collapse(2) schedule(static)
    for (int j = 0; j < P; ++j)
        for (int r = 0; r < P; ++r)
            memcpy((char*)out[j] + (int64_t)r * blk,
                   (const char*)x[r] + (int64_t)j * blk, (size_t)blk);
    return 0;
}

/* ---- AllToAllV (Table 2, variable-length AllToAll) ------------------ */

int orc_all_to_all_v(int P, const int64_t* C, int64_t row_bytes,
                     const void* const* x, void* const* out)
{
    if (orc_bad_p(P) || row_bytes < 1 || C == NULL)
        return -1;
    for (int e = 0; e < P * P; ++e)
        if (C[e] < 0)
            return -1;
    for (int r = 0; r < P; ++r) {
        for (int j = 0; j < P; ++j) {
            /* Source r's rows for j start after its rows for every j' < j. */
            int64_t src_row = 0;
            for (int jj = 0; jj < j; ++jj)
                src_row += C[r * P + jj];
            /* Destination j holds the rows of every r' < r before those of r. */
            int64_t dst_row = 0;
            for (int rr = 0; rr < r; ++rr)
                dst_row += C[rr * P + j];
            memcpy((char*)out[j] + dst_row * row_bytes,
                   (const char*)x[r] + src_row * row_bytes,
                   (size_t)(C[r * P + j] * row_bytes));
        }
    }
    return 0;
}

/* ---- AllReduce = AllGather(ReduceScatter(x)) (Figure 6) -------------- */

int orc_all_reduce(int P, int64_t n, int dtype, const void* const* x, void* const* out)
{
    if (orc_bad_p(P) || orc_bad_dtype(dtype) || n < 0)
        return -1;
    const int64_t esz = orc_esize(dtype);
    void* y[ORC_MAX_P];
    char* store = (char*)malloc((size_t)(P * n * esz) + 1);
    if (!store)
        return -2;
    for (int k = 0; k < P; ++k)
        y[k] = store + (int64_t)k * n * esz;
    int rc = orc_reduce_scatter(P, n, dtype, x, y);
    if (rc == 0)
        rc = orc_all_gather(P, n, esz, (const void* const*)y, out);
    free(store);
    return rc;
}

/* ---- variable-length ReduceScatter / AllGather (Table 2) ------------- */

int orc_reduce_scatter_v(int P, const int64_t* cnt, int dtype,
                         const void* const* x, void* const* y)
{
    if (orc_bad_p(P) || orc_bad_dtype(dtype) || cnt == NULL)
        return -1;
    int64_t off = 0;
    for (int k = 0; k < P; ++k) {
        if (cnt[k] < 0)
            return -1;
        const int64_t o = off;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < cnt[k]; ++i)
            orc_store(y[k], dtype, i, orc_sum_at(P, dtype, x, o + i));
        off += cnt[k];
    }
    return 0;
}

int orc_all_gather_v(int P, const int64_t* cnt, int64_t esize,
                     const void* const* z, void* const* out)
{
    if (orc_bad_p(P) || esize < 1 || cnt == NULL)
        return -1;
    for (int k = 0; k < P; ++k)
        if (cnt[k] < 0)
            return -1;
    for (int j = 0; j < P; ++j) {
        int64_t off = 0;
        for (int k = 0; k < P; ++k) {
            memcpy((char*)out[j] + off * esize, z[k], (size_t)(cnt[k] * esize));
            off += cnt[k];
        }
    }
    return 0;
}

/* ---- MoE dispatch and combine ---------------------------------------- */

static int orc_bad_moe(int P, int E, int k, int64_t T, const int32_t* const* ids)
{
    return orc_bad_p(P) || E < P || E % P != 0 || k < 1 || T < 0 || (T > 0 && !ids);
}

int orc_moe_route(int P, int E, int k, int64_t T, const int32_t* const* ids,
                  int32_t* const* pos, int32_t* counts, int64_t* recv)
{
    if (orc_bad_moe(P, E, k, T, ids) || !pos || !counts || !recv)
        return -1;
    const int per = E / P;
    const int64_t n = T * k;
    for (int r = 0; r < P; ++r)
        for (int64_t i = 0; i < n; ++i)
            pos[r][i] = -1;
    for (int j = 0; j < P; ++j) {
        int64_t row = 0;
        for (int e = j * per; e < (j + 1) * per; ++e)       /* experts in order */
            for (int r = 0; r < P; ++r) {                   /* sources in order */
                int32_t c = 0;
                for (int64_t i = 0; i < n; ++i)             /* entries in order */
                    if (ids[r][i] == e) {
                        pos[r][i] = (int32_t)row++;
                        ++c;
                    }
                counts[(int64_t)r * E + e] = c;
            }
        recv[j] = row;
    }
    return 0;
}

int orc_moe_dispatch(int P, int E, int k, int64_t T, const int32_t* const* ids,
                     const int32_t* const* pos, int64_t cap, int64_t row_bytes,
                     const void* const* x, void* const* out)
{
    if (orc_bad_moe(P, E, k, T, ids) || cap < 0 || row_bytes < 0)
        return -1;
    const int per = E / P;
    for (int r = 0; r < P; ++r)
        for (int64_t i = 0; i < T * k; ++i) {
            const int32_t e = ids[r][i];
            if (e < 0 || e >= E || pos[r][i] < 0 || pos[r][i] >= cap)
                continue;
            const int64_t t = i / k;
            memcpy((char*)out[e / per] + (int64_t)pos[r][i] * row_bytes,
                   (const char*)x[r] + t * row_bytes, (size_t)row_bytes);
        }
    return 0;
}

int orc_moe_combine(int P, int E, int k, int64_t T, const int32_t* const* ids,
                    const int32_t* const* pos, const float* const* w, int64_t cap,
                    int64_t H, int dtype, const void* const* y, void* const* out)
{
    if (orc_bad_moe(P, E, k, T, ids) || orc_bad_dtype(dtype) || cap < 0 || H < 0)
        return -1;
    const int per = E / P;
    for (int r = 0; r < P; ++r) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t h = 0; h < H; ++h) {
                float acc = 0.0f;
                for (int c = 0; c < k; ++c) {
                    const int64_t i = t * k + c;
                    const int32_t e = ids[r][i];
                    if (e < 0 || e >= E || pos[r][i] < 0 || pos[r][i] >= cap)
                        continue;
                    const float v = orc_load(y[e / per], dtype, (int64_t)pos[r][i] * H + h);
                    acc = fmaf(w[r][i], v, acc);
                }
                orc_store(out[r], dtype, t * H + h, acc);
            }
    }
    return 0;
}

int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int orc_set_threads(int n)
{
    if (n < 1)
        return 1;
#ifdef _OPENMP
    omp_set_num_threads(n);
#endif
    return 0;
}
