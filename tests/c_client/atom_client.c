/* A plain C program that uses libatom through include/atom.h alone, with
 * device memory from the HIP runtime: the ReduceScatter of P bf16 inputs
 * (zero-staging), then the AllGather of its outputs through SNAC (staged),
 * then the AllReduce of the same inputs through SNAC. Inputs are read from
 * a file of P * P * n bf16 values (input r at r * P * n); the three results
 * are written to one file in that order (P * n, then P * P * n twice).
 *
 * usage: atom_client P n inputs.bin outputs.bin
 * Exit status 0 on success; a message on stderr otherwise. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "atom.h"

#define FAIL(...)                                                                  \
    do {                                                                           \
        fprintf(stderr, __VA_ARGS__);                                              \
        fputc('\n', stderr);                                                       \
        exit(1);                                                                   \
    } while (0)

static void hip_ok(hipError_t e, const char* what)
{
    if (e != hipSuccess)
        FAIL("%s: %s", what, hipGetErrorString(e));
}

static void atom_ok(atom_status s, const char* what)
{
    if (s != ATOM_OK)
        FAIL("%s: %s", what, atom_status_string(s));
}

int main(int argc, char** argv)
{
    if (argc != 5)
        FAIL("usage: %s P n inputs.bin outputs.bin", argv[0]);
    const int P = atoi(argv[1]);
    const int64_t n = atoll(argv[2]);
    if (P < 1 || P > ATOM_MAX_RANKS || n < 1)
        FAIL("bad P or n");
    const size_t esz = 2;                              /* bf16 */
    const size_t in_elems = (size_t)P * (size_t)n;     /* per input */
    uint16_t* host_in = malloc(in_elems * P * esz);
    uint16_t* host_out = malloc((in_elems + 2 * in_elems * P) * esz);
    if (!host_in || !host_out)
        FAIL("host allocation");
    FILE* f = fopen(argv[3], "rb");
    if (!f || fread(host_in, esz, in_elems * P, f) != in_elems * P)
        FAIL("reading %s", argv[3]);
    fclose(f);

    void* x[ATOM_MAX_RANKS];     /* inputs, P * n each */
    void* y[ATOM_MAX_RANKS];     /* ReduceScatter outputs, n each */
    void* g[ATOM_MAX_RANKS];     /* AllGather outputs, P * n each */
    void* a[ATOM_MAX_RANKS];     /* AllReduce outputs, P * n each */
    for (int r = 0; r < P; ++r) {
        hip_ok(hipMalloc(&x[r], in_elems * esz), "hipMalloc x");
        hip_ok(hipMalloc(&y[r], (size_t)n * esz), "hipMalloc y");
        hip_ok(hipMalloc(&g[r], in_elems * esz), "hipMalloc g");
        hip_ok(hipMalloc(&a[r], in_elems * esz), "hipMalloc a");
        hip_ok(hipMemcpy(x[r], host_in + (size_t)r * in_elems, in_elems * esz, hipMemcpyHostToDevice),
               "hipMemcpy x");
    }

    atom_layout part = {ATOM_LAYOUT_PARTITIONED, P, x, n, NULL, 1, ATOM_DT_BF16};
    atom_layout shard_y = {ATOM_LAYOUT_SHARD, P, y, n, NULL, 1, ATOM_DT_BF16};
    atom_layout gath_g = {ATOM_LAYOUT_GATHERED, P, g, n, NULL, 1, ATOM_DT_BF16};
    atom_layout gath_a = {ATOM_LAYOUT_GATHERED, P, a, n, NULL, 1, ATOM_DT_BF16};
    atom_config staged = {0};
    staged.flags = ATOM_F_STAGED;

    atom_ok(atom_collective(&part, &shard_y, ATOM_OP_SUM, NULL, NULL), "ReduceScatter");
    atom_ok(atom_collective(&shard_y, &gath_g, ATOM_OP_COPY, &staged, NULL), "staged AllGather");
    atom_ok(atom_collective(&part, &gath_a, ATOM_OP_SUM, &staged, NULL), "staged AllReduce");
    atom_ok(atom_sync_status(NULL), "atom_sync_status");

    uint16_t* o = host_out;
    for (int r = 0; r < P; ++r, o += n)
        hip_ok(hipMemcpy(o, y[r], (size_t)n * esz, hipMemcpyDeviceToHost), "hipMemcpy y");
    for (int r = 0; r < P; ++r, o += in_elems)
        hip_ok(hipMemcpy(o, g[r], in_elems * esz, hipMemcpyDeviceToHost), "hipMemcpy g");
    for (int r = 0; r < P; ++r, o += in_elems)
        hip_ok(hipMemcpy(o, a[r], in_elems * esz, hipMemcpyDeviceToHost), "hipMemcpy a");
    f = fopen(argv[4], "wb");
    const size_t total = (size_t)P * n + 2 * in_elems * P;
    if (!f || fwrite(host_out, esz, total, f) != total)
        FAIL("writing %s", argv[4]);
    fclose(f);
    for (int r = 0; r < P; ++r) {
        hip_ok(hipFree(x[r]), "hipFree");
        hip_ok(hipFree(y[r]), "hipFree");
        hip_ok(hipFree(g[r]), "hipFree");
        hip_ok(hipFree(a[r]), "hipFree");
    }
    free(host_in);
    free(host_out);
    return 0;
}
