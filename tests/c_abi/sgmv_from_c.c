/* The library through its C ABI alone, from a C program: no Python, no
 * torch.  Device memory and the stream come from the HIP runtime API; the
 * reference is the CPU oracle (test infrastructure, linked only here).
 *
 * A float32 pool of 2 layers x 2 projections that read one input (h_in 256;
 * h_out 128 and 64), 6 adapters of ranks 3..32, 37 tokens in seeded segments
 * (some without an adapter), base outputs given:
 *   1. lora_pool_register from host arrays, lora_plan_create,
 *      lora_workspace_bytes, lora_plan_upload;
 *   2. sgmv_fused per layer over both projections; every output slice
 *      within the contract tolerance of the float64 oracle;
 *   3. sgmv_shrink + sgmv_expand through a device v give sgmv_fused's bits;
 *   4. a bad call (layer out of range) returns LORA_EINVAL with a message
 *      and enqueues nothing (y unchanged).
 * Prints one line per step; exit status 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lora_sgmv.h"

int oracle_delta_f64(int32_t T, int32_t h_in, int32_t h_out, const float *x, int64_t ldx,
                     int32_t S, const int32_t *seg_starts, const int32_t *seg_adapter,
                     int32_t n_adapters, const int32_t *adapter_ids, const int32_t *ranks,
                     const float *scales, const float *const *A, const float *const *B,
                     const float *y_in, int64_t ld_in, double *y_out, int64_t ld_out,
                     int32_t threads);

enum { L = 2, NP = 2, HIN = 256, T = 37, NA = 6, RMAX = 32, W = 192 };
static const int32_t H_OUT[NP] = {128, 64};
static const int32_t OFF[NP] = {0, 128};
static const int32_t RANK[NA] = {3, 8, 16, 13, 24, 32};

static uint64_t g_state = 0x9e3779b97f4a7c15ull;
static float uniform(void) {            /* a seeded draw in [-1, 1) */
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((double)(g_state >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                 \
            return 1;                                                                  \
        }                                                                              \
    } while (0)
#define LORA_OK_(call)                                                                 \
    do {                                                                               \
        lora_status s_ = (call);                                                       \
        if (s_ != LORA_OK) {                                                           \
            fprintf(stderr, "%s: status %d: %s\n", #call, (int)s_, lora_last_error()); \
            return 1;                                                                  \
        }                                                                              \
    } while (0)

int main(void) {
    /* adapters: A[a][p] = [L][rank][HIN], B[a][p] = [L][h_out][rank] */
    static float *A[NA][NP], *B[NA][NP];
    float scale[NA];
    for (int a = 0; a < NA; ++a) {
        scale[a] = 0.5f + 0.25f * (float)a;
        for (int p = 0; p < NP; ++p) {
            const size_t na = (size_t)L * RANK[a] * HIN, nb = (size_t)L * H_OUT[p] * RANK[a];
            A[a][p] = malloc(na * sizeof(float));
            B[a][p] = malloc(nb * sizeof(float));
            for (size_t i = 0; i < na; ++i) A[a][p][i] = uniform() / 16.0f;
            for (size_t i = 0; i < nb; ++i) B[a][p][i] = uniform() * 0.02f;
        }
    }
    /* segments: lengths 1..4, adapters -1..NA-1 */
    int32_t starts[T + 1], seg_ad[T];
    int32_t S = 0, t = 0;
    starts[0] = 0;
    while (t < T) {
        int32_t n = 1 + (int32_t)((uniform() + 1.0f) * 2.0f);
        if (t + n > T) n = T - t;
        seg_ad[S] = (int32_t)((uniform() + 1.0f) * 0.5f * (NA + 1)) - 1;
        if (seg_ad[S] >= NA) seg_ad[S] = NA - 1;
        t += n;
        starts[++S] = t;
    }
    static float x[L][T * HIN], base[L][T * W];
    for (int l = 0; l < L; ++l) {
        for (int i = 0; i < T * HIN; ++i) x[l][i] = uniform();
        for (int i = 0; i < T * W; ++i) base[l][i] = uniform();
    }

    /* 1. pool, adapters, plan, workspace */
    lora_pool_desc d;
    memset(&d, 0, sizeof d);
    d.num_layers = L;
    d.num_proj = NP;
    for (int p = 0; p < NP; ++p) { d.h_in[p] = HIN; d.h_out[p] = H_OUT[p]; }
    d.r_max = RMAX;
    d.rank_granule = 8;
    d.max_slots = NA;
    d.dtype = LORA_F32;
    uint64_t slab_bytes = 0;
    for (int a = 0; a < NA; ++a) slab_bytes += lora_pool_extent_bytes(&d, RANK[a]);
    void *slab = NULL;
    HIP_OK(hipMalloc(&slab, slab_bytes));
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    lora_pool *pool = NULL;
    LORA_OK_(lora_pool_create(&pool, &d, slab, slab_bytes));
    for (int a = 0; a < NA; ++a)
        LORA_OK_(lora_pool_register(pool, a, RANK[a], scale[a], (const void *const *)A[a],
                                    (const void *const *)B[a], 1, st));
    lora_plan *plan = NULL;
    LORA_OK_(lora_plan_create(&plan, pool, T, starts, seg_ad, S));
    const uint64_t ws_bytes = lora_workspace_bytes(pool, T, S, NP);
    if (ws_bytes < lora_plan_workspace_bytes(plan, NP)) {
        fprintf(stderr, "workspace bound %llu below the plan's need\n",
                (unsigned long long)ws_bytes);
        return 1;
    }
    void *ws = NULL;
    HIP_OK(hipMalloc(&ws, ws_bytes));
    LORA_OK_(lora_plan_upload(plan, ws, ws_bytes, NP, st));
    printf("C ABI: pool of %d adapters (%llu slab bytes), plan of %d segments, workspace %llu "
           "bytes\n", NA, (unsigned long long)slab_bytes, S, (unsigned long long)ws_bytes);

    /* 2. the fused call, checked against the oracle */
    const int32_t projs[NP] = {0, 1};
    float *dx, *dbase, *dy, *dy2, *dv;
    HIP_OK(hipMalloc((void **)&dx, sizeof(float) * T * HIN));
    HIP_OK(hipMalloc((void **)&dbase, sizeof(float) * T * W));
    HIP_OK(hipMalloc((void **)&dy, sizeof(float) * T * W));
    HIP_OK(hipMalloc((void **)&dy2, sizeof(float) * T * W));
    HIP_OK(hipMalloc((void **)&dv, sizeof(float) * T * NP * RMAX));
    static float y[T * W], y2[T * W];
    static double ref[T * 128];
    int32_t ids[NA];
    for (int a = 0; a < NA; ++a) ids[a] = a;
    double worst = 0.0;
    for (int l = 0; l < L; ++l) {
        HIP_OK(hipMemcpy(dx, x[l], sizeof(float) * T * HIN, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(dbase, base[l], sizeof(float) * T * W, hipMemcpyHostToDevice));
        LORA_OK_(sgmv_fused(pool, plan, l, NP, projs, OFF, dx, HIN, dbase, W, dy, W, st));
        HIP_OK(hipStreamSynchronize(st));
        HIP_OK(hipMemcpy(y, dy, sizeof(float) * T * W, hipMemcpyDeviceToHost));
        for (int p = 0; p < NP; ++p) {
            const float *Ap[NA], *Bp[NA];
            for (int a = 0; a < NA; ++a) {
                Ap[a] = A[a][p] + (size_t)l * RANK[a] * HIN;
                Bp[a] = B[a][p] + (size_t)l * H_OUT[p] * RANK[a];
            }
            if (oracle_delta_f64(T, HIN, H_OUT[p], x[l], HIN, S, starts, seg_ad, NA, ids, RANK,
                                 scale, Ap, Bp, base[l] + OFF[p], W, ref, H_OUT[p], 1)) {
                fprintf(stderr, "oracle failed\n");
                return 1;
            }
            double mref = 0.0, err = 0.0;
            for (int i = 0; i < T; ++i)
                for (int o = 0; o < H_OUT[p]; ++o) {
                    const double r = ref[i * H_OUT[p] + o];
                    mref = fmax(mref, fabs(r));
                    err = fmax(err, fabs((double)y[i * W + OFF[p] + o] - r));
                }
            const double tol = 1e-2 * mref + 1e-3;
            if (!(err <= tol)) {
                fprintf(stderr, "layer %d projection %d: max|diff| %.3e > %.3e\n", l, p, err, tol);
                return 1;
            }
            worst = fmax(worst, err / tol);
        }

        /* 3. shrink + expand through v: the fused call's bits */
        HIP_OK(hipMemcpy(dy2, base[l], sizeof(float) * T * W, hipMemcpyHostToDevice));
        HIP_OK(hipMemset(dv, 0, sizeof(float) * T * NP * RMAX));
        LORA_OK_(sgmv_shrink(pool, plan, l, NP, projs, dx, HIN, dv, NP * RMAX, st));
        LORA_OK_(sgmv_expand(pool, plan, l, NP, projs, OFF, dv, NP * RMAX, dy2, W, st));
        HIP_OK(hipStreamSynchronize(st));
        HIP_OK(hipMemcpy(y2, dy2, sizeof(float) * T * W, hipMemcpyDeviceToHost));
        if (memcmp(y, y2, sizeof y)) {
            fprintf(stderr, "layer %d: the two-step result differs from the fused one\n", l);
            return 1;
        }
    }
    printf("C ABI: sgmv_fused within the oracle's tolerance on %d layers x %d projections "
           "(worst %.2e of it); sgmv_shrink + sgmv_expand bit-identical\n", L, NP, worst);

    /* 4. a refused call enqueues nothing */
    HIP_OK(hipMemcpy(y2, dy, sizeof(float) * T * W, hipMemcpyDeviceToHost));
    const lora_status bad = sgmv_fused(pool, plan, L, NP, projs, OFF, dx, HIN, dbase, W, dy, W,
                                       st);
    HIP_OK(hipStreamSynchronize(st));
    HIP_OK(hipMemcpy(y, dy, sizeof(float) * T * W, hipMemcpyDeviceToHost));
    if (bad != LORA_EINVAL || !lora_last_error()[0] || memcmp(y, y2, sizeof y)) {
        fprintf(stderr, "a call with layer %d returned %d and %s y\n", L, (int)bad,
                memcmp(y, y2, sizeof y) ? "changed" : "kept");
        return 1;
    }
    printf("C ABI: layer %d refused with LORA_EINVAL (\"%s\"), y unchanged\n", L,
           lora_last_error());

    LORA_OK_(lora_plan_destroy(plan));
    LORA_OK_(lora_pool_destroy(pool));
    HIP_OK(hipFree(ws));
    HIP_OK(hipFree(slab));
    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(dbase));
    HIP_OK(hipFree(dy));
    HIP_OK(hipFree(dy2));
    HIP_OK(hipFree(dv));
    HIP_OK(hipStreamDestroy(st));
    for (int a = 0; a < NA; ++a)
        for (int p = 0; p < NP; ++p) { free(A[a][p]); free(B[a][p]); }
    printf("C ABI: all checks passed\n");
    return 0;
}
