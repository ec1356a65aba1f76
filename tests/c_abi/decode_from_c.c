/*
 * decode_from_c.c -- the paged decode library driven from plain C99, with no
 * Python or torch in the process: device buffers from the HIP runtime API,
 * every kernel family through pa_decode_plan / pa_decode_ex, the output
 * compared with the fp64 oracle (oracle/pa_oracle.c, test infrastructure).
 *
 * Checked mode (PA_CHECK=1, pa_config.check): an out-of-range block id in a
 * used table entry, or a length past the table, is rejected with
 * PA_ERR_DEVICE_CHECK before any attention kernel runs (the output buffer
 * keeps its fill pattern), pa_get_device_error reports it once, and good
 * inputs still decode correctly.
 *
 * Test program only: built by the package build step, run by
 * tests/test_c_abi.py on a GPU.  Exit status 0 when every case is within the
 * bound, 1 on a mismatch, 2 on an API or HIP error.
 */
#define _POSIX_C_SOURCE 200112L   /* setenv / unsetenv */

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "pa_decode.h"

/* oracle/pa_oracle.c */
int oracle_decode(const void *query, const void *key_cache, const void *value_cache,
                  const int32_t *block_tables, const int32_t *seq_lens, double scale, double *out,
                  int S, int Hq, int Hkv, int D, int B, int NB, int max_blocks, int dtype,
                  const int32_t *rows, int nrows);
enum { ORACLE_BF16 = 2 };

#define HIP_OK(x)                                                            \
    do {                                                                     \
        hipError_t e_ = (x);                                                 \
        if (e_ != hipSuccess) {                                              \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));          \
            exit(2);                                                         \
        }                                                                    \
    } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

static uint32_t next_u32(void) {   /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545f4914f6cdd1dull) >> 32);
}

static float next_uniform(void) { return (float)next_u32() / 4294967296.0f * 2.0f - 1.0f; }

/* float -> bfloat16, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

enum { S = 5, HQ = 16, HKV = 4, D = 128, B = 16, MAX_BLOCKS = 64 };
static const int lens[S] = {1, 33, 300, 1000, 0};

/* max over elements of |got - ref| / max(|ref|, 1e-2 * max over the row |ref|) */
static double max_rel_err(const float *got, const double *ref) {
    double worst = 0.0;
    for (int r = 0; r < S * HQ; ++r) {
        double rowmax = 0.0;
        for (int d = 0; d < D; ++d) rowmax = fmax(rowmax, fabs(ref[r * D + d]));
        for (int d = 0; d < D; ++d) {
            const double e = ref[r * D + d], g = got[r * D + d];
            const double den = fmax(fabs(e), 1e-2 * rowmax);
            const double rel = den > 0.0 ? fabs(g - e) / den : fabs(g - e);
            if (!(rel <= worst)) worst = isnan(rel) ? INFINITY : fmax(worst, rel);
        }
    }
    return worst;
}

/* 1 if every byte of the device output still holds the 0xff fill */
static int output_untouched(void *dout, float *got) {
    HIP_OK(hipMemcpy(got, dout, sizeof(float) * S * HQ * D, hipMemcpyDeviceToHost));
    const unsigned char *bytes = (const unsigned char *)got;
    for (size_t i = 0; i < sizeof(float) * S * HQ * D; ++i)
        if (bytes[i] != 0xff) return 0;
    return 1;
}

static int checked_mode(void *dq, void *dk, void *dv, void *dt, void *dl, void *dout,
                        const int32_t *tables, int NB, float scale, const double *ref,
                        float *got) {
    int failed = 0;
    pa_plan plan;
    if (pa_decode_plan(S, HQ, HKV, D, B, NB, MAX_BLOCKS, PA_BF16, PA_F32, NULL, &plan) != PA_OK)
        return 1;
    void *ws = NULL, *dt_bad, *dl_bad;
    if (plan.workspace_bytes) HIP_OK(hipMalloc(&ws, plan.workspace_bytes));
    HIP_OK(hipMalloc(&dt_bad, sizeof(int32_t) * S * MAX_BLOCKS));
    HIP_OK(hipMalloc(&dl_bad, sizeof(int32_t) * S));
    int32_t *bad_tables = malloc(sizeof(int32_t) * S * MAX_BLOCKS);
    memcpy(bad_tables, tables, sizeof(int32_t) * S * MAX_BLOCKS);
    bad_tables[3 * MAX_BLOCKS + 5] = NB + 3;      /* sequence 3 (1000 tokens) uses entry 5 */
    bad_tables[1 * MAX_BLOCKS + 7] = -9;          /* sequence 1 (33 tokens) never reads entry 7 */
    HIP_OK(hipMemcpy(dt_bad, bad_tables, sizeof(int32_t) * S * MAX_BLOCKS, hipMemcpyHostToDevice));
    int32_t bad_lens[S];
    memcpy(bad_lens, lens, sizeof bad_lens);
    bad_lens[2] = MAX_BLOCKS * B + 1;             /* longer than the table */
    HIP_OK(hipMemcpy(dl_bad, bad_lens, sizeof bad_lens, hipMemcpyHostToDevice));

    /* PA_CHECK=1: the bad id is rejected and nothing runs */
    setenv("PA_CHECK", "1", 1);
    HIP_OK(hipMemset(dout, 0xff, sizeof(float) * S * HQ * D));
    pa_status st = pa_decode(dq, dk, dv, dt_bad, dl, scale, dout, S, HQ, HKV, D, B, NB,
                             MAX_BLOCKS, PA_BF16, PA_F32, ws, plan.workspace_bytes, NULL);
    int untouched = output_untouched(dout, got);
    int32_t first = 0;
    pa_status dev = pa_get_device_error(NULL, &first);
    int32_t first2 = 0;
    pa_status dev2 = pa_get_device_error(NULL, &first2);
    int ok = st == PA_ERR_DEVICE_CHECK && untouched && dev == PA_ERR_DEVICE_CHECK && first == 3 &&
             dev2 == PA_OK && first2 == -1;
    printf("checked mode, bad block id: %s, output untouched %d, device error %s (first %d), "
           "then %s: %s\n", pa_status_string(st), untouched, pa_status_string(dev), (int)first,
           pa_status_string(dev2), ok ? "ok" : "FAIL");
    failed |= !ok;

    /* PA_CHECK=1 and good inputs: a normal, correct call */
    HIP_OK(hipMemset(dout, 0xff, sizeof(float) * S * HQ * D));
    st = pa_decode(dq, dk, dv, dt, dl, scale, dout, S, HQ, HKV, D, B, NB, MAX_BLOCKS, PA_BF16,
                   PA_F32, ws, plan.workspace_bytes, NULL);
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got, dout, sizeof(float) * S * HQ * D, hipMemcpyDeviceToHost));
    double worst = max_rel_err(got, ref);
    dev = pa_get_device_error(NULL, &first);
    ok = st == PA_OK && worst <= 2e-3 && dev == PA_OK;
    printf("checked mode, good inputs: %s, rel err %.3e, device error %s: %s\n",
           pa_status_string(st), worst, pa_status_string(dev), ok ? "ok" : "FAIL");
    failed |= !ok;

    /* the environment off, pa_config.check = 1: a length past the table */
    unsetenv("PA_CHECK");
    const pa_config on = {PA_KERNEL_AUTO, 0, 0, 0, 1, 0};
    HIP_OK(hipMemset(dout, 0xff, sizeof(float) * S * HQ * D));
    st = pa_decode_ex(dq, dk, dv, dt, dl_bad, scale, dout, S, HQ, HKV, D, B, NB, MAX_BLOCKS,
                      PA_BF16, PA_F32, &on, ws, plan.workspace_bytes, NULL);
    untouched = output_untouched(dout, got);
    dev = pa_get_device_error(NULL, &first);
    ok = st == PA_ERR_DEVICE_CHECK && untouched && dev == PA_ERR_DEVICE_CHECK && first == 2;
    printf("config check, bad length: %s, output untouched %d, first %d: %s\n",
           pa_status_string(st), untouched, (int)first, ok ? "ok" : "FAIL");
    failed |= !ok;

    /* PA_CHECK=1 but pa_config.check = -1: unchecked, good inputs */
    setenv("PA_CHECK", "1", 1);
    const pa_config off = {PA_KERNEL_AUTO, 0, 0, 0, -1, 0};
    st = pa_decode_ex(dq, dk, dv, dt, dl, scale, dout, S, HQ, HKV, D, B, NB, MAX_BLOCKS,
                      PA_BF16, PA_F32, &off, ws, plan.workspace_bytes, NULL);
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got, dout, sizeof(float) * S * HQ * D, hipMemcpyDeviceToHost));
    worst = max_rel_err(got, ref);
    ok = st == PA_OK && worst <= 2e-3;
    printf("config check off under PA_CHECK=1: %s, rel err %.3e: %s\n", pa_status_string(st),
           worst, ok ? "ok" : "FAIL");
    failed |= !ok;
    unsetenv("PA_CHECK");

    if (ws) HIP_OK(hipFree(ws));
    HIP_OK(hipFree(dt_bad));
    HIP_OK(hipFree(dl_bad));
    free(bad_tables);
    return failed;
}

int main(void) {
    int used = 0;
    for (int s = 0; s < S; ++s) used += (lens[s] + B - 1) / B;
    const int NB = used + 8;
    const size_t pool_elems = (size_t)NB * HKV * B * D;
    uint16_t *q = malloc(sizeof(uint16_t) * S * HQ * D);
    uint16_t *kc = malloc(sizeof(uint16_t) * pool_elems);
    uint16_t *vc = malloc(sizeof(uint16_t) * pool_elems);
    int32_t *tables = malloc(sizeof(int32_t) * S * MAX_BLOCKS);
    int32_t *perm = malloc(sizeof(int32_t) * NB);
    double *ref = malloc(sizeof(double) * S * HQ * D);
    float *got = malloc(sizeof(float) * S * HQ * D);
    for (size_t i = 0; i < (size_t)S * HQ * D; ++i) q[i] = to_bf16(next_uniform());
    for (size_t i = 0; i < pool_elems; ++i) kc[i] = to_bf16(next_uniform());
    for (size_t i = 0; i < pool_elems; ++i) vc[i] = to_bf16(next_uniform());
    for (int i = 0; i < NB; ++i) perm[i] = i;
    for (int i = NB - 1; i > 0; --i) {   /* shuffled physical blocks */
        const int j = (int)(next_u32() % (uint32_t)(i + 1));
        const int32_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
    int next = 0;
    for (int s = 0; s < S; ++s) {
        const int n = (lens[s] + B - 1) / B;
        for (int j = 0; j < MAX_BLOCKS; ++j) tables[s * MAX_BLOCKS + j] = j < n ? perm[next + j] : 0;
        next += n;
    }
    const float scale = 1.0f / sqrtf((float)D);
    if (oracle_decode(q, kc, vc, tables, lens, scale, ref, S, HQ, HKV, D, B, NB, MAX_BLOCKS,
                      ORACLE_BF16, NULL, S * HQ) != 0) {
        fprintf(stderr, "oracle rejected the inputs\n");
        return 2;
    }

    void *dq, *dk, *dv, *dt, *dl, *dout;
    HIP_OK(hipMalloc(&dq, sizeof(uint16_t) * S * HQ * D));
    /* 8 spare blocks past the NB the calls declare: the checked-mode case's
     * out-of-range id (NB + 3) stays inside the allocation */
    const size_t alloc_elems = pool_elems + (size_t)8 * HKV * B * D;
    HIP_OK(hipMalloc(&dk, sizeof(uint16_t) * alloc_elems));
    HIP_OK(hipMalloc(&dv, sizeof(uint16_t) * alloc_elems));
    HIP_OK(hipMemset(dk, 0, sizeof(uint16_t) * alloc_elems));
    HIP_OK(hipMemset(dv, 0, sizeof(uint16_t) * alloc_elems));
    HIP_OK(hipMalloc(&dt, sizeof(int32_t) * S * MAX_BLOCKS));
    HIP_OK(hipMalloc(&dl, sizeof(int32_t) * S));
    HIP_OK(hipMalloc(&dout, sizeof(float) * S * HQ * D));
    HIP_OK(hipMemcpy(dq, q, sizeof(uint16_t) * S * HQ * D, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dk, kc, sizeof(uint16_t) * pool_elems, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, vc, sizeof(uint16_t) * pool_elems, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dt, tables, sizeof(int32_t) * S * MAX_BLOCKS, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dl, lens, sizeof(int32_t) * S, hipMemcpyHostToDevice));

    /* an argument error comes back as a status, before any launch */
    const pa_status bad = pa_decode(NULL, dk, dv, dt, dl, scale, dout, S, HQ, HKV, D, B, NB,
                                    MAX_BLOCKS, PA_BF16, PA_F32, NULL, 0, NULL);
    printf("NULL query -> %s\n", pa_status_string(bad));
    if (bad != PA_ERR_NULL) return 1;

    const struct { int kernel, part, waves; const char *name; } cases[] = {
        {PA_KERNEL_AUTO, 0, 0, "auto"},        {PA_KERNEL_GENERIC, 0, 0, "generic"},
        {PA_KERNEL_VALU, 64, 0, "valu/split"}, {PA_KERNEL_MFMA, 0, 0, "mfma"},
        {PA_KERNEL_MFMA, 96, 0, "mfma/split"}, {PA_KERNEL_VALU, 256, 2, "valu/2 waves"},
        {PA_KERNEL_MFMA, 512, 4, "mfma/4 waves"},
    };
    int failed = 0;
    for (size_t c = 0; c < sizeof(cases) / sizeof(cases[0]); ++c) {
        const pa_config cfg = {cases[c].kernel, cases[c].part, 0, 0, 0, cases[c].waves};
        pa_plan plan;
        pa_status st = pa_decode_plan(S, HQ, HKV, D, B, NB, MAX_BLOCKS, PA_BF16, PA_F32, &cfg, &plan);
        if (st != PA_OK) {
            fprintf(stderr, "%s: plan: %s\n", cases[c].name, pa_status_string(st));
            return 2;
        }
        if (cases[c].waves && plan.token_waves != cases[c].waves) {
            fprintf(stderr, "%s: plan runs %d waves per item\n", cases[c].name, plan.token_waves);
            return 2;
        }
        void *ws = NULL;
        if (plan.workspace_bytes) HIP_OK(hipMalloc(&ws, plan.workspace_bytes));
        HIP_OK(hipMemset(dout, 0xff, sizeof(float) * S * HQ * D));   /* NaN until written */
        st = pa_decode_ex(dq, dk, dv, dt, dl, scale, dout, S, HQ, HKV, D, B, NB, MAX_BLOCKS,
                          PA_BF16, PA_F32, &cfg, ws, plan.workspace_bytes, NULL);
        if (st != PA_OK) {
            fprintf(stderr, "%s: decode: %s\n", cases[c].name, pa_status_string(st));
            return 2;
        }
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(got, dout, sizeof(float) * S * HQ * D, hipMemcpyDeviceToHost));
        if (ws) HIP_OK(hipFree(ws));
        /* |got - ref| <= 2e-3 * max(|ref|, 1e-2 * max over the row |ref|) */
        const double worst = max_rel_err(got, ref);
        const int ok = worst <= 2e-3;
        printf("%-12s kernel %d partition %5d split %d waves %d: max rel err %.3e %s\n",
               cases[c].name, plan.kernel, plan.partition_tokens, plan.split, plan.token_waves,
               worst, ok ? "ok" : "FAIL");
        failed |= !ok;
    }
    failed |= checked_mode(dq, dk, dv, dt, dl, dout, tables, NB, scale, ref, got);
    hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dt); hipFree(dl); hipFree(dout);
    free(q); free(kc); free(vc); free(tables); free(perm); free(ref); free(got);
    return failed ? 1 : 0;
}
