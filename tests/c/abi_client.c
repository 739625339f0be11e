/*
 * abi_client.c -- a plain C99 caller of libpa, with no Python or torch in the
 * process: device memory comes from the HIP runtime, every call goes through
 * include/pa.h.  It fills a small token-granular pool (3 requests, 8 query
 * heads over 2 KV heads, head_dim 128, 1024 slots) with deterministic bf16
 * values, plans once and runs decode twice (with and without lse), and
 * writes the inputs and outputs to the file named on the command line for a
 * test to check against the fp64 oracle.  Test infrastructure.
 *
 * Output file (little-endian): int32 B, Hq, Hkv, D, slots, entries; then
 * q (uint16 bf16 bits, B*Hq*D), K and V pools (slots*Hkv*D each), kv_indptr
 * (int32, B+1), kv_indices (int32, entries), out (float32, B*Hq*D), lse
 * (float32, B*Hq), and out of the run without lse (float32, B*Hq*D).
 * Exit status 0 on success; a failing call is named on stderr.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "pa.h"

enum { NB = 3, HQ = 8, HKV = 2, HD = 128, NSLOTS = 1024 };

#define CHECK_PA(call)                                                                          \
    do {                                                                                        \
        pa_status st_ = (call);                                                                 \
        if (st_ != PA_OK) {                                                                     \
            fprintf(stderr, "%s: %s (%s)\n", #call, pa_strerror(st_), pa_last_error_detail()); \
            return 1;                                                                           \
        }                                                                                       \
    } while (0)
#define CHECK_HIP(call)                                                       \
    do {                                                                      \
        hipError_t e_ = (call);                                               \
        if (e_ != hipSuccess) {                                               \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));        \
            return 1;                                                         \
        }                                                                     \
    } while (0)

/* a linear congruential sequence mapped to [-2, 2), rounded to bf16 (nearest even) */
static uint32_t lcg_state = 12345u;
static uint16_t next_bf16(void)
{
    lcg_state = lcg_state * 1664525u + 1013904223u;
    const float x = (float)(lcg_state >> 8) * (1.0f / 16777216.0f) * 4.0f - 2.0f;
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static int write_all(FILE *f, const void *p, size_t bytes)
{
    return fwrite(p, 1, bytes, f) == bytes ? 0 : 1;
}

int main(int argc, char **argv)
{
    if (argc != 2) {
        fprintf(stderr, "usage: %s OUTPUT_FILE\n", argv[0]);
        return 2;
    }
    const int32_t lengths[NB] = {1, 37, 300};
    int32_t indptr[NB + 1] = {0};
    for (int b = 0; b < NB; b++)
        indptr[b + 1] = indptr[b] + lengths[b];
    const int32_t entries = indptr[NB];
    int32_t *indices = malloc(sizeof(int32_t) * (size_t)entries);
    const size_t q_n = (size_t)NB * HQ * HD, pool_n = (size_t)NSLOTS * HKV * HD;
    uint16_t *q = malloc(q_n * 2), *k = malloc(pool_n * 2), *v = malloc(pool_n * 2);
    float *out = malloc(q_n * 4), *out2 = malloc(q_n * 4), *lse = malloc((size_t)NB * HQ * 4);
    if (!indices || !q || !k || !v || !out || !out2 || !lse) {
        fprintf(stderr, "host allocation failed\n");
        return 1;
    }
    for (int32_t j = 0; j < entries; j++)
        indices[j] = (int32_t)(((int64_t)j * 389 + 11) % NSLOTS);   /* distinct: 389 is odd */
    for (size_t i = 0; i < q_n; i++)
        q[i] = next_bf16();
    for (size_t i = 0; i < pool_n; i++)
        k[i] = next_bf16();
    for (size_t i = 0; i < pool_n; i++)
        v[i] = next_bf16();

    void *d_q, *d_k, *d_v, *d_idx, *d_out, *d_out2, *d_lse;
    CHECK_HIP(hipMalloc(&d_q, q_n * 2));
    CHECK_HIP(hipMalloc(&d_k, pool_n * 2));
    CHECK_HIP(hipMalloc(&d_v, pool_n * 2));
    CHECK_HIP(hipMalloc(&d_idx, sizeof(int32_t) * (size_t)entries));
    CHECK_HIP(hipMalloc(&d_out, q_n * 4));
    CHECK_HIP(hipMalloc(&d_out2, q_n * 4));
    CHECK_HIP(hipMalloc(&d_lse, (size_t)NB * HQ * 4));
    CHECK_HIP(hipMemcpy(d_q, q, q_n * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_k, k, pool_n * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_v, v, pool_n * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_idx, indices, sizeof(int32_t) * (size_t)entries, hipMemcpyHostToDevice));

    pa_plan_t *plan = NULL;
    CHECK_PA(pa_plan_create(&plan, NB, entries, 0, HQ, HKV, HD));
    CHECK_PA(pa_plan(plan, indptr, NULL, NB, 0, NULL));
    const float scale = 0.08838834764831845f;   /* 1/sqrt(128) */
    CHECK_PA(pa_decode_run(plan, d_q, d_k, d_v, NSLOTS, 0, (const int32_t *)d_idx, scale,
                           (float *)d_out, (float *)d_lse, NULL));
    CHECK_PA(pa_decode_run(plan, d_q, d_k, d_v, NSLOTS, 0, (const int32_t *)d_idx, scale,
                           (float *)d_out2, NULL, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(out, d_out, q_n * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(out2, d_out2, q_n * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(lse, d_lse, (size_t)NB * HQ * 4, hipMemcpyDeviceToHost));
    pa_plan_destroy(plan);

    FILE *f = fopen(argv[1], "wb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", argv[1]);
        return 1;
    }
    const int32_t header[6] = {NB, HQ, HKV, HD, NSLOTS, entries};
    int bad = write_all(f, header, sizeof header) | write_all(f, q, q_n * 2) | write_all(f, k, pool_n * 2) |
              write_all(f, v, pool_n * 2) | write_all(f, indptr, sizeof indptr) |
              write_all(f, indices, sizeof(int32_t) * (size_t)entries) | write_all(f, out, q_n * 4) |
              write_all(f, lse, (size_t)NB * HQ * 4) | write_all(f, out2, q_n * 4);
    bad |= fclose(f) != 0;
    if (bad) {
        fprintf(stderr, "writing %s failed\n", argv[1]);
        return 1;
    }
    CHECK_HIP(hipFree(d_q));
    CHECK_HIP(hipFree(d_k));
    CHECK_HIP(hipFree(d_v));
    CHECK_HIP(hipFree(d_idx));
    CHECK_HIP(hipFree(d_out));
    CHECK_HIP(hipFree(d_out2));
    CHECK_HIP(hipFree(d_lse));
    free(indices);
    free(q);
    free(k);
    free(v);
    free(out);
    free(out2);
    free(lse);
    printf("abi_client: %d requests, %d entries decoded\n", NB, entries);
    return 0;
}
