/*
 * The library used from C alone, through include/dit.h: device buffers from the
 * HIP runtime, calls into libdit.so, results checked on the host against
 * closed forms of the operations (no Python, no torch, no oracle). Prints one
 * line per check; exit status 0 when every check passes. The argument checks run
 * first and need no GPU (the library validates arguments before it touches the
 * device); without a GPU the program stops after them.
 *
 * Closed forms used ("Por que e absurdamente dificil gerar um filme inteiro
 * usando IA", section "Matematica por tras"; "DiT, Flow Matching e 3D
 * Attention", sections "A ruptura da U-Net" and "Flow Matching e Rectified
 * Flow"):
 *   - attention rows are convex combinations: v = 1 everywhere gives o = 1;
 *   - identical keys give equal weights: o = the mean of the sequence's v rows;
 *   - modulate with gamma = 0 gives y = beta;
 *   - an Euler step with dt = 0 leaves z unchanged.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dit.h"

static uint16_t to_bf16(float f) {   /* round to nearest even */
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}
static uint32_t g_rng = 12345u;
static float uniform_pm1(void) {   /* LCG, values in [-1, 1) */
    g_rng = g_rng * 1664525u + 1013904223u;
    return (float)(g_rng >> 8) * (2.0f / 16777216.0f) - 1.0f;
}

static int g_fail = 0;
static void report(const char* name, int ok, double err) {
    printf("%-44s %s (max err %.3g)\n", name, ok ? "ok" : "FAILED", err);
    if (!ok) g_fail = 1;
}

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));         \
            return 2;                                                                 \
        }                                                                             \
    } while (0)

int main(void) {
    enum { T = 300, H = 2, D = 128, N = T * H * D };
    printf("libdit version %d\n", dit_version());

    /* argument validation, before any device work: fake 16-byte-aligned device
       addresses that the library never dereferences on the host */
    {
        void* fq = (void*)(uintptr_t)0x100000;
        void* fk = (void*)(uintptr_t)0x200000;
        void* fv = (void*)(uintptr_t)0x300000;
        void* fo = (void*)(uintptr_t)0x400000;
        int rc = dit_attn3d(fo, fq, fk, fv, T, 3, 96, NULL, 1, 0, DIT_BF16, NULL);
        report("head_dim 96 rejected (DIT_E_UNSUPPORTED)", rc == DIT_E_UNSUPPORTED && dit_last_error()[0] != 0, 0.0);
        rc = dit_attn3d(fo, fq, fk, NULL, T, H, D, NULL, 1, 0, DIT_BF16, NULL);
        report("NULL v rejected (DIT_E_INVAL)", rc == DIT_E_INVAL, 0.0);
        rc = dit_attn3d(fq, fq, fk, fv, T, H, D, NULL, 1, 0, DIT_BF16, NULL);
        report("o overlapping q rejected (DIT_E_INVAL)", rc == DIT_E_INVAL, 0.0);
        rc = dit_rope3d(fq, fk, T, H, D, 1, 10, 30, NULL, 1, 44, 42, 40, 10000.0f, NULL, DIT_BF16, NULL);
        report("RoPE split not summing to head_dim rejected", rc == DIT_E_INVAL, 0.0);
        rc = dit_adaln_modulate(fo, fq, (const float*)fk, (const float*)fv, T, D, 7, 1e-6f, DIT_BF16, NULL);
        report("tokens not a multiple of tokens_per_row rejected", rc == DIT_E_INVAL, 0.0);
    }
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
        printf("no GPU: device checks skipped\n");
        return g_fail;
    }

    uint16_t* hq = malloc(N * 2);
    uint16_t* hk = malloc(N * 2);
    uint16_t* hv = malloc(N * 2);
    uint16_t* ho = malloc(N * 2);
    if (!hq || !hk || !hv || !ho) return 2;
    void *q, *k, *v, *o;
    HIP_OK(hipMalloc(&q, N * 2));
    HIP_OK(hipMalloc(&k, N * 2));
    HIP_OK(hipMalloc(&v, N * 2));
    HIP_OK(hipMalloc(&o, N * 2));

    int rc;
    /* v = 1: every output element is 1 */
    for (int i = 0; i < N; ++i) {
        hq[i] = to_bf16(2.0f * uniform_pm1());
        hk[i] = to_bf16(2.0f * uniform_pm1());
        hv[i] = to_bf16(1.0f);
    }
    HIP_OK(hipMemcpy(q, hq, N * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k, hk, N * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v, hv, N * 2, hipMemcpyHostToDevice));
    rc = dit_attn3d(o, q, k, v, T, H, D, NULL, 1, 0, DIT_BF16, NULL);
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(ho, o, N * 2, hipMemcpyDeviceToHost));
    double err = 0.0;
    for (int i = 0; i < N; ++i) err = fmax(err, fabs(from_bf16(ho[i]) - 1.0));
    report("attention, v = 1 gives o = 1", rc == DIT_OK && err <= 1.0 / 256, err);

    /* identical keys: o = mean of v over the sequence, for every query */
    for (int t = 1; t < T; ++t) memcpy(hk + (size_t)t * H * D, hk, H * D * 2);
    for (int i = 0; i < N; ++i) hv[i] = to_bf16(uniform_pm1());
    HIP_OK(hipMemcpy(k, hk, N * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v, hv, N * 2, hipMemcpyHostToDevice));
    rc = dit_attn3d(o, q, k, v, T, H, D, NULL, 1, 0, DIT_BF16, NULL);
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(ho, o, N * 2, hipMemcpyDeviceToHost));
    err = 0.0;
    for (int h = 0; h < H; ++h)
        for (int d = 0; d < D; ++d) {
            double mean = 0.0;
            for (int t = 0; t < T; ++t) mean += from_bf16(hv[((size_t)t * H + h) * D + d]);
            mean /= T;
            for (int t = 0; t < T; ++t) err = fmax(err, fabs(from_bf16(ho[((size_t)t * H + h) * D + d]) - mean));
        }
    report("attention, identical keys give mean(v)", rc == DIT_OK && err <= 2e-2, err);

    /* modulate with gamma = 0: y = beta (rows of 2 tokens) */
    {
        enum { TM = 64, DM = 256, ROWS = 32 };
        uint16_t* hx = malloc(TM * DM * 2);
        uint16_t* hy = malloc(TM * DM * 2);
        float* hb = malloc(ROWS * DM * 4);
        if (!hx || !hy || !hb) return 2;
        for (int i = 0; i < TM * DM; ++i) hx[i] = to_bf16(uniform_pm1());
        for (int i = 0; i < ROWS * DM; ++i) hb[i] = 0.25f * uniform_pm1();
        void *x, *y, *g, *b;
        HIP_OK(hipMalloc(&x, TM * DM * 2));
        HIP_OK(hipMalloc(&y, TM * DM * 2));
        HIP_OK(hipMalloc(&g, ROWS * DM * 4));
        HIP_OK(hipMalloc(&b, ROWS * DM * 4));
        HIP_OK(hipMemcpy(x, hx, TM * DM * 2, hipMemcpyHostToDevice));
        HIP_OK(hipMemset(g, 0, ROWS * DM * 4));
        HIP_OK(hipMemcpy(b, hb, ROWS * DM * 4, hipMemcpyHostToDevice));
        rc = dit_adaln_modulate(y, x, (const float*)g, (const float*)b, TM, DM, TM / ROWS, 1e-6f, DIT_BF16, NULL);
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(hy, y, TM * DM * 2, hipMemcpyDeviceToHost));
        int exact = 1;
        for (int t = 0; t < TM; ++t)
            for (int c = 0; c < DM; ++c)
                exact &= hy[t * DM + c] == to_bf16(hb[(t / (TM / ROWS)) * DM + c]);
        report("modulate, gamma = 0 gives y = beta (exact)", rc == DIT_OK && exact, 0.0);

        /* Euler with dt = 0: z unchanged, bit for bit (x as z, y as u) */
        void *z_out, *dt;
        HIP_OK(hipMalloc(&z_out, TM * DM * 2));
        HIP_OK(hipMalloc(&dt, ROWS * 4));
        HIP_OK(hipMemset(dt, 0, ROWS * 4));
        rc = rf_euler_step(z_out, x, y, (const float*)dt, TM, DM, TM / ROWS, DIT_BF16, NULL);
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(hy, z_out, TM * DM * 2, hipMemcpyDeviceToHost));
        report("Euler, dt = 0 leaves z unchanged (exact)", rc == DIT_OK && memcmp(hy, hx, TM * DM * 2) == 0, 0.0);
        hipFree(x); hipFree(y); hipFree(g); hipFree(b); hipFree(z_out); hipFree(dt);
        free(hx); free(hy); free(hb);
    }
    hipFree(q); hipFree(k); hipFree(v); hipFree(o);
    free(hq); free(hk); free(hv); free(ho);
    printf(g_fail ? "FAILED\n" : "all checks passed\n");
    return g_fail;
}
