/*
 * CPU oracle for the multi-adapter LoRA delta.  TEST INFRASTRUCTURE ONLY:
 * tests, the smoke check and the benchmark's CPU-baseline leg may call it;
 * the product path never does, and nothing here is shared with the GPU
 * library (no headers, helpers or tables in common).
 *
 * What it computes, per token t of a heterogeneous batch:
 *
 *   y[t] = y_in[t] + s_i * B_i (A_i x[t]),   i = adapter of the segment holding t
 *
 * - LoRA keeps the base weight W frozen and adds a low-rank update made of
 *   two small trained matrices A and B ("TGI Multi-LoRA: Deploy Once, Serve
 *   30 Models", section "Technical Foundation: Low-Rank Adaptation").  Here
 *   A_i is r_i x h_in and B_i is h_out x r_i, so B_i A_i has W's shape.
 * - Each request names one adapter, so one batch mixes adapters ("How
 *   Multi-LoRA Serving Works" on the same page); segments are contiguous
 *   token ranges that share an adapter, the grouping SGMV exploits ("Compress
 *   then Serve", rebuttal paragraph on Punica's segmented gather).
 * - The rank-R intermediate v = A_i x[t] is formed in float32 with A at
 *   scale 1, and then s_i B_i v is added into the token's slice of y
 *   ("Compress then Serve", the rebuttal's pseudocode of the delta).  y_in
 *   is whatever y held before the call (zero, W x, or a given base output).
 *
 * Plain definition, written out: no blocking, no reordering.  Sums run in
 * ascending index order.  oracle_delta_f32 accumulates in float (the
 * precision the pages fix for the intermediate buffer); oracle_delta_f64
 * accumulates in double and is used to measure the float version's own
 * rounding.  Built with -O2 -ffp-contract=off and no fast-math so the
 * sequential order and the separate multiply and add are kept.
 *
 * Readings where the pages are silent: adapter id -1 means "no adapter"
 * (the token keeps y_in); an id that is not in the adapter table, or a
 * segment table that does not partition [0, T), is an error (return -1).
 *
 * Two more functions follow the same loops: the delta of jointly
 * compressed adapters (oracle_delta_sigma_*: a shared basis and a per-
 * segment core between the A and B steps) and the weighted merge of several
 * adapters per request (oracle_delta_merge_*).
 *
 * Parity pins: every function here is pinned by the tests listed in the
 * oracle's test module (B = 0 identity, merged-weight equality, rank-1
 * closed form, permutation and split invariance, padding invariance,
 * linearity, indicator adapters, a hand-computed example; for the cores:
 * identity cores give plain LoRA bit for bit, power-of-two diagonal cores
 * equal scaled A rows bit for bit, full cores equal s (B Sigma A) x in
 * float64; for merges: one slot is plain LoRA, slots apply in order, the
 * merge equals x (sum_k w_k s_k B_k A_k)^T in float64).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static int check_segments(int32_t T, int32_t S, const int32_t *seg_starts)
{
    if (T < 0 || S < 0) return -1;
    if (seg_starts[0] != 0 || seg_starts[S] != T) return -1;
    for (int32_t s = 0; s < S; ++s)
        if (seg_starts[s + 1] < seg_starts[s]) return -1;
    return 0;
}

/* Index of adapter `id` in the table, or -1. A plain linear search. */
static int32_t find_adapter(int32_t n, const int32_t *ids, int32_t id)
{
    for (int32_t a = 0; a < n; ++a)
        if (ids[a] == id) return a;
    return -1;
}

/*
 * Expand the segment table into the per-token adapter table index (the
 * per-token `indices` form of the same batch): tok_a[t] = index into the
 * adapter table, or -1 for "no adapter".  Returns 0 or -1.
 */
static int token_adapters(int32_t T, int32_t S, const int32_t *seg_starts,
                          const int32_t *seg_adapter, int32_t n_adapters,
                          const int32_t *adapter_ids, int32_t *tok_a)
{
    if (check_segments(T, S, seg_starts)) return -1;
    for (int32_t s = 0; s < S; ++s) {
        int32_t a = -1;
        if (seg_adapter[s] != -1) {
            a = find_adapter(n_adapters, adapter_ids, seg_adapter[s]);
            if (a < 0) return -1;
        }
        for (int32_t t = seg_starts[s]; t < seg_starts[s + 1]; ++t) tok_a[t] = a;
    }
    return 0;
}

static int32_t max_rank(int32_t n, const int32_t *ranks)
{
    int32_t r = 1;
    for (int32_t a = 0; a < n; ++a)
        if (ranks[a] > r) r = ranks[a];
    return r;
}

/*
 * Arguments (all host memory, row-major):
 *   T, h_in, h_out      token rows, input width, output width
 *   x [T][ldx]          activations (float32; bf16 inputs are passed widened)
 *   S, seg_starts[S+1], seg_adapter[S]   the segment table
 *   n_adapters, adapter_ids[n], ranks[n], scales[n]
 *   A[n] -> [rank][h_in], B[n] -> [h_out][rank]   per-adapter weights
 *   y_in [T][ld_in] or NULL (zero)
 *   y_out [T][ld_out]   result
 *   threads             OpenMP threads over tokens (<= 1: sequential)
 * Returns 0, or -1 for a malformed segment table or an unknown adapter id.
 */
int oracle_delta_f32(int32_t T, int32_t h_in, int32_t h_out,
                     const float *x, int64_t ldx,
                     int32_t S, const int32_t *seg_starts, const int32_t *seg_adapter,
                     int32_t n_adapters, const int32_t *adapter_ids,
                     const int32_t *ranks, const float *scales,
                     const float *const *A, const float *const *B,
                     const float *y_in, int64_t ld_in,
                     float *y_out, int64_t ld_out, int32_t threads)
{
    int32_t *tok_a = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    if (!tok_a) return -1;
    if (token_adapters(T, S, seg_starts, seg_adapter, n_adapters, adapter_ids, tok_a)) {
        free(tok_a);
        return -1;
    }
    const int32_t r_big = max_rank(n_adapters, ranks);

#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 1 ? threads : 1)
    for (int32_t t = 0; t < T; ++t) {
        float v[r_big];
        float *yt = y_out + (int64_t)t * ld_out;
        for (int32_t o = 0; o < h_out; ++o)
            yt[o] = y_in ? y_in[(int64_t)t * ld_in + o] : 0.0f;
        const int32_t a = tok_a[t];
        if (a < 0) continue;
        const int32_t r = ranks[a];
        const float sc = scales[a];
        const float *xt = x + (int64_t)t * ldx;
        /* A step (scale 1): v = A_i x[t] */
        for (int32_t j = 0; j < r; ++j) {
            float acc = 0.0f;
            const float *aj = A[a] + (int64_t)j * h_in;
            for (int32_t k = 0; k < h_in; ++k) acc += aj[k] * xt[k];
            v[j] = acc;
        }
        /* B step: y[t] += s_i * (B_i v) */
        for (int32_t o = 0; o < h_out; ++o) {
            float d = 0.0f;
            const float *bo = B[a] + (int64_t)o * r;
            for (int32_t j = 0; j < r; ++j) d += bo[j] * v[j];
            yt[o] = yt[o] + sc * d;
        }
    }
    free(tok_a);
    return 0;
}

/* The same loop with double accumulation; y_out is double. */
int oracle_delta_f64(int32_t T, int32_t h_in, int32_t h_out,
                     const float *x, int64_t ldx,
                     int32_t S, const int32_t *seg_starts, const int32_t *seg_adapter,
                     int32_t n_adapters, const int32_t *adapter_ids,
                     const int32_t *ranks, const float *scales,
                     const float *const *A, const float *const *B,
                     const float *y_in, int64_t ld_in,
                     double *y_out, int64_t ld_out, int32_t threads)
{
    int32_t *tok_a = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    if (!tok_a) return -1;
    if (token_adapters(T, S, seg_starts, seg_adapter, n_adapters, adapter_ids, tok_a)) {
        free(tok_a);
        return -1;
    }
    const int32_t r_big = max_rank(n_adapters, ranks);

#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 1 ? threads : 1)
    for (int32_t t = 0; t < T; ++t) {
        double v[r_big];
        double *yt = y_out + (int64_t)t * ld_out;
        for (int32_t o = 0; o < h_out; ++o)
            yt[o] = y_in ? (double)y_in[(int64_t)t * ld_in + o] : 0.0;
        const int32_t a = tok_a[t];
        if (a < 0) continue;
        const int32_t r = ranks[a];
        const double sc = (double)scales[a];
        const float *xt = x + (int64_t)t * ldx;
        for (int32_t j = 0; j < r; ++j) {
            double acc = 0.0;
            const float *aj = A[a] + (int64_t)j * h_in;
            for (int32_t k = 0; k < h_in; ++k) acc += (double)aj[k] * (double)xt[k];
            v[j] = acc;
        }
        for (int32_t o = 0; o < h_out; ++o) {
            double d = 0.0;
            const float *bo = B[a] + (int64_t)o * r;
            for (int32_t j = 0; j < r; ++j) d += (double)bo[j] * v[j];
            yt[o] = yt[o] + sc * d;
        }
    }
    free(tok_a);
    return 0;
}

/*
 * Jointly compressed adapters:
 *
 *   y[t] = y_in[t] + s_i * B_c u,   u = Sigma_j v,   v = A_c x[t]
 *
 * with v and u in float32 ("Compress then Serve", the rebuttal's pseudocode
 * of the delta with a per-adapter core: the shared A, then the core, then
 * the shared B with the scale into the y slice).  A_c and B_c are the shared
 * basis of the segment's entry c in the adapter table (a cluster, r x h_in
 * and h_out x r); Sigma_j is the segment's core, r x r (kind 2, "JD-Full")
 * or its diagonal of r values (kind 1, "JD-Diag"); seg_sigma[s] = -1 means
 * no core (Sigma = identity), which is plain LoRA.  sigma[j] points at core
 * j, row-major with row length sigma_ld (kind 2).  Same loops, order and
 * error returns as oracle_delta_f32; also -1 for a core index out of range.
 */
int oracle_delta_sigma_f32(int32_t T, int32_t h_in, int32_t h_out,
                           const float *x, int64_t ldx,
                           int32_t S, const int32_t *seg_starts, const int32_t *seg_adapter,
                           const int32_t *seg_sigma,
                           int32_t n_adapters, const int32_t *adapter_ids,
                           const int32_t *ranks, const float *scales,
                           const float *const *A, const float *const *B,
                           int32_t n_sigma, int32_t sigma_kind, const float *const *sigma,
                           int64_t sigma_ld,
                           const float *y_in, int64_t ld_in,
                           float *y_out, int64_t ld_out, int32_t threads)
{
    if (sigma_kind != 1 && sigma_kind != 2) return -1;
    int32_t *tok_a = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    int32_t *tok_s = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    if (!tok_a || !tok_s) { free(tok_a); free(tok_s); return -1; }
    if (token_adapters(T, S, seg_starts, seg_adapter, n_adapters, adapter_ids, tok_a)) {
        free(tok_a); free(tok_s);
        return -1;
    }
    for (int32_t s = 0; s < S; ++s) {
        if (seg_sigma[s] < -1 || seg_sigma[s] >= n_sigma) { free(tok_a); free(tok_s); return -1; }
        for (int32_t t = seg_starts[s]; t < seg_starts[s + 1]; ++t) tok_s[t] = seg_sigma[s];
    }
    const int32_t r_big = max_rank(n_adapters, ranks);

#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 1 ? threads : 1)
    for (int32_t t = 0; t < T; ++t) {
        float v[r_big], u[r_big];
        float *yt = y_out + (int64_t)t * ld_out;
        for (int32_t o = 0; o < h_out; ++o)
            yt[o] = y_in ? y_in[(int64_t)t * ld_in + o] : 0.0f;
        const int32_t a = tok_a[t];
        if (a < 0) continue;
        const int32_t r = ranks[a];
        const float sc = scales[a];
        const float *xt = x + (int64_t)t * ldx;
        /* v = A_c x[t] */
        for (int32_t j = 0; j < r; ++j) {
            float acc = 0.0f;
            const float *aj = A[a] + (int64_t)j * h_in;
            for (int32_t k = 0; k < h_in; ++k) acc += aj[k] * xt[k];
            v[j] = acc;
        }
        /* u = Sigma_j v (u = v without a core) */
        const int32_t sj = tok_s[t];
        for (int32_t j = 0; j < r; ++j) {
            if (sj < 0) {
                u[j] = v[j];
            } else if (sigma_kind == 1) {
                u[j] = sigma[sj][j] * v[j];
            } else {
                float acc = 0.0f;
                const float *row = sigma[sj] + (int64_t)j * sigma_ld;
                for (int32_t k = 0; k < r; ++k) acc += row[k] * v[k];
                u[j] = acc;
            }
        }
        /* y[t] += s * (B_c u) */
        for (int32_t o = 0; o < h_out; ++o) {
            float d = 0.0f;
            const float *bo = B[a] + (int64_t)o * r;
            for (int32_t j = 0; j < r; ++j) d += bo[j] * u[j];
            yt[o] = yt[o] + sc * d;
        }
    }
    free(tok_a);
    free(tok_s);
    return 0;
}

/* The same with double accumulation; y_out is double. */
int oracle_delta_sigma_f64(int32_t T, int32_t h_in, int32_t h_out,
                           const float *x, int64_t ldx,
                           int32_t S, const int32_t *seg_starts, const int32_t *seg_adapter,
                           const int32_t *seg_sigma,
                           int32_t n_adapters, const int32_t *adapter_ids,
                           const int32_t *ranks, const float *scales,
                           const float *const *A, const float *const *B,
                           int32_t n_sigma, int32_t sigma_kind, const float *const *sigma,
                           int64_t sigma_ld,
                           const float *y_in, int64_t ld_in,
                           double *y_out, int64_t ld_out, int32_t threads)
{
    if (sigma_kind != 1 && sigma_kind != 2) return -1;
    int32_t *tok_a = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    int32_t *tok_s = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    if (!tok_a || !tok_s) { free(tok_a); free(tok_s); return -1; }
    if (token_adapters(T, S, seg_starts, seg_adapter, n_adapters, adapter_ids, tok_a)) {
        free(tok_a); free(tok_s);
        return -1;
    }
    for (int32_t s = 0; s < S; ++s) {
        if (seg_sigma[s] < -1 || seg_sigma[s] >= n_sigma) { free(tok_a); free(tok_s); return -1; }
        for (int32_t t = seg_starts[s]; t < seg_starts[s + 1]; ++t) tok_s[t] = seg_sigma[s];
    }
    const int32_t r_big = max_rank(n_adapters, ranks);

#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 1 ? threads : 1)
    for (int32_t t = 0; t < T; ++t) {
        double v[r_big], u[r_big];
        double *yt = y_out + (int64_t)t * ld_out;
        for (int32_t o = 0; o < h_out; ++o)
            yt[o] = y_in ? (double)y_in[(int64_t)t * ld_in + o] : 0.0;
        const int32_t a = tok_a[t];
        if (a < 0) continue;
        const int32_t r = ranks[a];
        const double sc = (double)scales[a];
        const float *xt = x + (int64_t)t * ldx;
        for (int32_t j = 0; j < r; ++j) {
            double acc = 0.0;
            const float *aj = A[a] + (int64_t)j * h_in;
            for (int32_t k = 0; k < h_in; ++k) acc += (double)aj[k] * (double)xt[k];
            v[j] = acc;
        }
        const int32_t sj = tok_s[t];
        for (int32_t j = 0; j < r; ++j) {
            if (sj < 0) {
                u[j] = v[j];
            } else if (sigma_kind == 1) {
                u[j] = (double)sigma[sj][j] * v[j];
            } else {
                double acc = 0.0;
                const float *row = sigma[sj] + (int64_t)j * sigma_ld;
                for (int32_t k = 0; k < r; ++k) acc += (double)row[k] * v[k];
                u[j] = acc;
            }
        }
        for (int32_t o = 0; o < h_out; ++o) {
            double d = 0.0;
            const float *bo = B[a] + (int64_t)o * r;
            for (int32_t j = 0; j < r; ++j) d += (double)bo[j] * u[j];
            yt[o] = yt[o] + sc * d;
        }
    }
    free(tok_a);
    free(tok_s);
    return 0;
}

/*
 * Weighted merging of adapters per request ("predibase/lorax" listing:
 * adapters merged per request into a weighted ensemble): segment s carries
 * K slots (adapter seg_adapters[s*K + k], weight seg_weights[s*K + k]), and
 *
 *   y[t] = y_in[t] + sum_k (w_k * s_k) * B_k (A_k x[t])
 *
 * summed slot by slot in k order (the product w_k * s_k rounded to float
 * first), each slot's delta as in oracle_delta_f32.  Reading: the merge is
 * linear in the adapters' deltas (the same as merging their low-rank
 * updates B A with those weights); a slot with adapter -1 adds nothing.
 * Returns -1 for a malformed segment table or an unknown adapter id.
 */
int oracle_delta_merge_f32(int32_t T, int32_t h_in, int32_t h_out,
                           const float *x, int64_t ldx,
                           int32_t S, const int32_t *seg_starts, int32_t K,
                           const int32_t *seg_adapters, const float *seg_weights,
                           int32_t n_adapters, const int32_t *adapter_ids,
                           const int32_t *ranks, const float *scales,
                           const float *const *A, const float *const *B,
                           const float *y_in, int64_t ld_in,
                           float *y_out, int64_t ld_out, int32_t threads)
{
    if (K < 1 || check_segments(T, S, seg_starts)) return -1;
    int32_t *slot_a = (int32_t *)malloc(sizeof(int32_t) * (size_t)(S * K > 0 ? S * K : 1));
    if (!slot_a) return -1;
    for (int32_t i = 0; i < S * K; ++i) {
        slot_a[i] = -1;
        if (seg_adapters[i] != -1) {
            slot_a[i] = find_adapter(n_adapters, adapter_ids, seg_adapters[i]);
            if (slot_a[i] < 0) { free(slot_a); return -1; }
        }
    }
    const int32_t r_big = max_rank(n_adapters, ranks);

#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 1 ? threads : 1)
    for (int32_t s = 0; s < S; ++s) {
        for (int32_t t = seg_starts[s]; t < seg_starts[s + 1]; ++t) {
            float v[r_big];
            float *yt = y_out + (int64_t)t * ld_out;
            for (int32_t o = 0; o < h_out; ++o)
                yt[o] = y_in ? y_in[(int64_t)t * ld_in + o] : 0.0f;
            const float *xt = x + (int64_t)t * ldx;
            for (int32_t k = 0; k < K; ++k) {
                const int32_t a = slot_a[s * K + k];
                if (a < 0) continue;
                const int32_t r = ranks[a];
                const float sw = seg_weights[s * K + k] * scales[a];
                for (int32_t j = 0; j < r; ++j) {
                    float acc = 0.0f;
                    const float *aj = A[a] + (int64_t)j * h_in;
                    for (int32_t kk = 0; kk < h_in; ++kk) acc += aj[kk] * xt[kk];
                    v[j] = acc;
                }
                for (int32_t o = 0; o < h_out; ++o) {
                    float d = 0.0f;
                    const float *bo = B[a] + (int64_t)o * r;
                    for (int32_t j = 0; j < r; ++j) d += bo[j] * v[j];
                    yt[o] = yt[o] + sw * d;
                }
            }
        }
    }
    free(slot_a);
    return 0;
}

/* The same merge with double accumulation; y_out is double. */
int oracle_delta_merge_f64(int32_t T, int32_t h_in, int32_t h_out,
                           const float *x, int64_t ldx,
                           int32_t S, const int32_t *seg_starts, int32_t K,
                           const int32_t *seg_adapters, const float *seg_weights,
                           int32_t n_adapters, const int32_t *adapter_ids,
                           const int32_t *ranks, const float *scales,
                           const float *const *A, const float *const *B,
                           const float *y_in, int64_t ld_in,
                           double *y_out, int64_t ld_out, int32_t threads)
{
    if (K < 1 || check_segments(T, S, seg_starts)) return -1;
    int32_t *slot_a = (int32_t *)malloc(sizeof(int32_t) * (size_t)(S * K > 0 ? S * K : 1));
    if (!slot_a) return -1;
    for (int32_t i = 0; i < S * K; ++i) {
        slot_a[i] = -1;
        if (seg_adapters[i] != -1) {
            slot_a[i] = find_adapter(n_adapters, adapter_ids, seg_adapters[i]);
            if (slot_a[i] < 0) { free(slot_a); return -1; }
        }
    }
    const int32_t r_big = max_rank(n_adapters, ranks);

#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 1 ? threads : 1)
    for (int32_t s = 0; s < S; ++s) {
        for (int32_t t = seg_starts[s]; t < seg_starts[s + 1]; ++t) {
            double v[r_big];
            double *yt = y_out + (int64_t)t * ld_out;
            for (int32_t o = 0; o < h_out; ++o)
                yt[o] = y_in ? (double)y_in[(int64_t)t * ld_in + o] : 0.0;
            const float *xt = x + (int64_t)t * ldx;
            for (int32_t k = 0; k < K; ++k) {
                const int32_t a = slot_a[s * K + k];
                if (a < 0) continue;
                const int32_t r = ranks[a];
                const double sw = (double)seg_weights[s * K + k] * (double)scales[a];
                for (int32_t j = 0; j < r; ++j) {
                    double acc = 0.0;
                    const float *aj = A[a] + (int64_t)j * h_in;
                    for (int32_t kk = 0; kk < h_in; ++kk) acc += (double)aj[kk] * (double)xt[kk];
                    v[j] = acc;
                }
                for (int32_t o = 0; o < h_out; ++o) {
                    double d = 0.0;
                    const float *bo = B[a] + (int64_t)o * r;
                    for (int32_t j = 0; j < r; ++j) d += (double)bo[j] * v[j];
                    yt[o] = yt[o] + sw * d;
                }
            }
        }
    }
    free(slot_a);
    return 0;
}
