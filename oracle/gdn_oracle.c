/*
 * Parity oracle for the gated delta rule scan -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library. The product path (the HIP library and its
 * Python binding) never calls it, and the two share no code.
 *
 * What it computes: the plain sequential definition of the gated delta rule,
 * one token at a time, in float64. For every (sequence b, value head h):
 *
 *     S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t (scale * q_t)
 *
 * S is dv x dk (row i = value dimension, column j = key dimension). That
 * orientation is the one of the tinygrad gated-delta reference loops (the
 * state is contracted with a key vector over its last index) on the
 * "27b 935/47" compare page (tests of gated_delta_decode and
 * gated_delta_prefill in test_llm_quant_cpu.py); the output is read from
 * the updated state, as in the same tests, where the core output equals
 * alpha*S*q + delta*(k.q) with S the state before the update.
 *
 * The decay enters as g (log-decay) and alpha = exp(g): a padded step with
 * g = 0 and beta = 0 leaves S unchanged (the no-op rule in the commit log of
 * the page "mergable fast RDNA3 Qwen 3.6", symbolic-length prefill entry).
 *
 * Key heads are shared by value heads: head_map 0 ("tiled") reads key head
 * h % Hk, the repeat of key heads that gdn_qkv performs in the gdn_qkv test on
 * the "27b 935/47" page; head_map 1 ("grouped") reads key head h / (Hv / Hk).
 *
 * Inputs are float32 (bfloat16 inputs arrive already widened exactly); every
 * operation is done in double. Threads split the independent (b, h) pairs
 * only, so results are bit-identical for any thread count.
 *
 * Parity pins (tests/test_oracle_pins.py): dense brute-force unrolling,
 * exact rational arithmetic on tiny inputs, the pages' one-step formula,
 * the padded no-op rule, continuation splits, the beta = 0 closed form,
 * delta-rule recall with orthonormal keys, scale linearity, head-map
 * permutation and thread-count invariance; for the gated RMSNorm epilogue
 * (gdn_oracle_gated_rmsnorm, at the end), unit root-mean-square rows, the eps
 * closed form, quoted sigmoid values and per-column weights; for the
 * per-channel decay (gdn_oracle_kda_*, at the end), agreement with the scalar
 * rule when all channels decay alike, the beta = 0 closed form per channel,
 * dense unrolling, one-hot recall with per-channel forgetting, continuation
 * and decode-equals-prefill, bit for bit.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int key_head_of(int h, int Hk, int Hv, int head_map) {
    if (head_map == 0) return h % Hk;
    return h / (Hv / Hk);
}

/* One token of the recurrence on a dv x dk row-major state, then the output. */
static void oracle_step(double *S, int dk, int dv, double alpha, double beta, double scale,
                        const float *qq, const float *kk, const float *vv, double *u, double *out) {
    /* u = S k */
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * (double)kk[j];
        u[i] = acc;
    }
    /* S <- alpha * S (I - beta k k^T) + beta v k^T
     *    = alpha * (S - beta (S k) k^T) + beta v k^T                    */
    for (int i = 0; i < dv; ++i) {
        for (int j = 0; j < dk; ++j) {
            double kj = (double)kk[j];
            double s = S[(int64_t)i * dk + j];
            S[(int64_t)i * dk + j] = alpha * (s - beta * u[i] * kj) + beta * (double)vv[i] * kj;
        }
    }
    /* o = S (scale q), from the updated state */
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * (scale * (double)qq[j]);
        out[i] = acc;
    }
}

static int check_shape(int B, int T, int Hk, int Hv, int dk, int dv, int head_map) {
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1 || dk < 1 || dv < 1) return 1;
    if (Hv % Hk != 0) return 1;
    if (head_map != 0 && head_map != 1) return 1;
    return 0;
}

/*
 * Prefill: q, k [B][Hk][T][dk]; v [B][Hv][T][dv]; g, beta [B][Hv][T];
 * s0 [B][Hv][dv][dk] in double (a float32 initial state widens exactly) or NULL (zero state).
 * pairs: list of flattened (b * Hv + h) indices to compute, or NULL for all
 * B*Hv pairs in order. Outputs are compact over the list:
 * o [npairs][T][dv], s_final [npairs][dv][dk] (either may be NULL).
 * Returns 0, or 1 on invalid arguments.
 */
int gdn_oracle_prefill(int B, int T, int Hk, int Hv, int dk, int dv, int head_map, double scale,
                       const float *q, const float *k, const float *v,
                       const float *g, const float *beta, const double *s0,
                       const int64_t *pairs, int64_t npairs,
                       double *o, double *s_final, int nthreads) {
    if (check_shape(B, T, Hk, Hv, dk, dv, head_map)) return 1;
    if (!pairs) npairs = (int64_t)B * Hv;
    for (int64_t p = 0; pairs && p < npairs; ++p)
        if (pairs[p] < 0 || pairs[p] >= (int64_t)B * Hv) return 1;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
    for (int64_t p = 0; p < npairs; ++p) {
        int64_t pair = pairs ? pairs[p] : p;
        int b = (int)(pair / Hv), h = (int)(pair % Hv);
        int kh = key_head_of(h, Hk, Hv, head_map);
        double *S = (double *)calloc((size_t)dv * dk, sizeof(double));
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *out = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !u || !out) { bad = 1; free(S); free(u); free(out); continue; }
        if (s0) {
            const double *src = s0 + ((int64_t)b * Hv + h) * dv * dk;
            for (int64_t e = 0; e < (int64_t)dv * dk; ++e) S[e] = src[e];
        }
        for (int t = 0; t < T; ++t) {
            const float *qq = q + (((int64_t)b * Hk + kh) * T + t) * dk;
            const float *kk = k + (((int64_t)b * Hk + kh) * T + t) * dk;
            const float *vv = v + (((int64_t)b * Hv + h) * T + t) * dv;
            int64_t gi = ((int64_t)b * Hv + h) * T + t;
            double alpha = exp((double)g[gi]);
            oracle_step(S, dk, dv, alpha, (double)beta[gi], scale, qq, kk, vv, u, out);
            if (o) memcpy(o + ((int64_t)p * T + t) * dv, out, sizeof(double) * (size_t)dv);
        }
        if (s_final) memcpy(s_final + (int64_t)p * dv * dk, S, sizeof(double) * (size_t)dv * dk);
        free(S); free(u); free(out);
    }
    return bad ? 2 : 0;
}

/*
 * One decode step for a batch: q, k [B][Hk][dk]; v [B][Hv][dv]; g, beta [B][Hv].
 * state [npairs][dv][dk] (float64, updated in place) and o [npairs][dv] are
 * compact over the pair list (NULL = all B*Hv pairs in order).
 */
int gdn_oracle_decode(int B, int Hk, int Hv, int dk, int dv, int head_map, double scale,
                      const float *q, const float *k, const float *v,
                      const float *g, const float *beta,
                      const int64_t *pairs, int64_t npairs,
                      double *state, double *o, int nthreads) {
    if (check_shape(B, 1, Hk, Hv, dk, dv, head_map)) return 1;
    if (!state || !o) return 1;
    if (!pairs) npairs = (int64_t)B * Hv;
    for (int64_t p = 0; pairs && p < npairs; ++p)
        if (pairs[p] < 0 || pairs[p] >= (int64_t)B * Hv) return 1;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(| : bad)
    for (int64_t p = 0; p < npairs; ++p) {
        int64_t pair = pairs ? pairs[p] : p;
        int b = (int)(pair / Hv), h = (int)(pair % Hv);
        int kh = key_head_of(h, Hk, Hv, head_map);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!u) { bad = 1; continue; }
        const float *qq = q + ((int64_t)b * Hk + kh) * dk;
        const float *kk = k + ((int64_t)b * Hk + kh) * dk;
        const float *vv = v + ((int64_t)b * Hv + h) * dv;
        double alpha = exp((double)g[pair]);
        oracle_step(state + (int64_t)p * dv * dk, dk, dv, alpha, (double)beta[pair], scale,
                    qq, kk, vv, u, o + (int64_t)p * dv);
        free(u);
    }
    return bad ? 2 : 0;
}

int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Gated RMSNorm of output rows: the output epilogue of the gated delta kernels
 * on the "27b 935/47" page (the q8_gated_rmsnorm test, and the norm_weight /
 * norm_eps arguments of gated_delta, whose result is checked against an
 * RMSNorm of the core output). For each row x of n values:
 *
 *     y = x / sqrt(mean(x^2) + eps) * weight * silu(gate),  silu(z) = z / (1 + exp(-z))
 *
 * with the gate factor left out when gate is NULL. weight has n values shared
 * by every row (the page applies weight[:128] to both heads of its core
 * output). Rows are independent; x and y may be the same array.
 */
int gdn_oracle_gated_rmsnorm(int64_t rows, int n, const double *x, const float *gate, const float *weight,
                             double eps, double *y, int nthreads) {
    if (rows < 0 || n <= 0 || !x || !weight || !y || !(eps >= 0.0)) return 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * n;
        double ss = 0.0;
        for (int i = 0; i < n; ++i) ss += xr[i] * xr[i];
        const double inv = 1.0 / sqrt(ss / n + eps);
        double *yr = y + r * n;
        for (int i = 0; i < n; ++i) {
            double v = xr[i] * inv * (double)weight[i];
            if (gate) {
                const double z = (double)gate[r * n + i];
                v *= z / (1.0 + exp(-z));
            }
            yr[i] = v;
        }
    }
    return 0;
}

/*
 * Input prologue of the scan: the causal depthwise convolution with SiLU and
 * the gdn_qkv split of the "27b 935/47" page (its causal_conv_silu and
 * gdn_qkv tests). x holds, per (b, t), Cch = (2 Hk + Hv) d channels; conv
 * weight w is [Cch][K]; the convolution state holds the K - 1 rows before
 * t = 0. With window = state rows followed by the rows of x:
 *
 *     y[b][t][c] = silu(sum_{i<K} window[b][t + i][c] * w[c][i])
 *
 * Channels [0, Hk d) are q, [Hk d, 2 Hk d) are k and the rest v, each split
 * into heads of d channels. q and k heads are scaled by
 * 1 / sqrt(sum of squares over the head + eps) (an L2 normalisation); v is
 * left as is. Outputs are head-major: q, k [B][Hk][T][d], v [B][Hv][T][d].
 * The value heads' sharing of key heads is left to the scan (no repeat), and
 * so is the 1/sqrt(d) query scale. state_out (if not NULL) receives the last
 * K - 1 window rows, the state that continues the sequence; it may be
 * state_in. state_in NULL means zero rows.
 */
int gdn_oracle_qkv_prologue(int B, int T, int Hk, int Hv, int d, int K, const float *x, const float *w,
                            const double *state_in, double *q, double *k, double *v, double *state_out,
                            double eps, int nthreads) {
    if (B <= 0 || T < 0 || Hk <= 0 || Hv <= 0 || d <= 0 || K <= 0 || !x || !w || !q || !k || !v) return 1;
    if (d > 1024) return 3;
    const int C = (2 * Hk + Hv) * d;
    const int W = T + K - 1;
    double *win = (double *)malloc(sizeof(double) * (size_t)W * C);
    double *newst = state_out ? (double *)malloc(sizeof(double) * (size_t)B * (K - 1) * C) : NULL;
    if (!win || (state_out && !newst)) {
        free(win);
        free(newst);
        return 2;
    }
    for (int b = 0; b < B; ++b) {
        for (int r = 0; r < K - 1; ++r)
            for (int c = 0; c < C; ++c)
                win[(size_t)r * C + c] = state_in ? state_in[((size_t)b * (K - 1) + r) * C + c] : 0.0;
        for (int t = 0; t < T; ++t)
            for (int c = 0; c < C; ++c) win[(size_t)(t + K - 1) * C + c] = (double)x[((size_t)b * T + t) * C + c];
        if (newst)
            for (int r = 0; r < K - 1; ++r)
                for (int c = 0; c < C; ++c) newst[((size_t)b * (K - 1) + r) * C + c] = win[(size_t)(T + r) * C + c];
#ifdef _OPENMP
        if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
        for (int t = 0; t < T; ++t) {
            double y[1024];  /* one head (d <= 1024) */
            for (int hh = 0; hh < 2 * Hk + Hv; ++hh) {
                for (int j = 0; j < d; ++j) {
                    const int c = hh * d + j;
                    double acc = 0.0;
                    for (int i = 0; i < K; ++i) acc += win[(size_t)(t + i) * C + c] * (double)w[(size_t)c * K + i];
                    y[j] = acc / (1.0 + exp(-acc));
                }
                double f = 1.0;
                if (hh < 2 * Hk) {
                    double ss = 0.0;
                    for (int j = 0; j < d; ++j) ss += y[j] * y[j];
                    f = 1.0 / sqrt(ss + eps);
                }
                double *dst = hh < Hk ? q + (((size_t)b * Hk + hh) * T + t) * d
                            : hh < 2 * Hk ? k + (((size_t)b * Hk + (hh - Hk)) * T + t) * d
                                          : v + (((size_t)b * Hv + (hh - 2 * Hk)) * T + t) * d;
                for (int j = 0; j < d; ++j) dst[j] = y[j] * f;
            }
        }
    }
    if (newst) {
        memcpy(state_out, newst, sizeof(double) * (size_t)B * (K - 1) * C);
        free(newst);
    }
    free(win);
    return 0;
}

/*
 * Per-channel decay (the KDA variant: the "channel decay" of the Kimi K3 experiments on the
 * "master..kimi_slop" page, which keeps one decay value per key channel instead of one per
 * head). The pages give no formula; the plain reading used here replaces the scalar decay
 * exp(g_t) of the gated delta rule by a diagonal matrix over the key channels:
 *
 *     S_t = S_{t-1} diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t (scale * q_t)
 *
 * with g_t a vector of dk log-decays. S is dv x dk as above, so the decay scales the key
 * columns of S. With every channel of g_t equal it is the gated delta rule.
 */
static void oracle_kda_step(double *S, int dk, int dv, const double *alpha, double beta, double scale,
                            const float *qq, const float *kk, const float *vv, double *u, double *out) {
    /* S <- S diag(alpha) */
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j) S[(int64_t)i * dk + j] *= alpha[j];
    /* u = S k (of the decayed state) */
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * (double)kk[j];
        u[i] = acc;
    }
    /* S <- S (I - beta k k^T) + beta v k^T = S + beta (v - S k) k^T */
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j) S[(int64_t)i * dk + j] += beta * ((double)vv[i] - u[i]) * (double)kk[j];
    /* o = S (scale q), from the updated state */
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * (scale * (double)qq[j]);
        out[i] = acc;
    }
}

/*
 * KDA prefill: as gdn_oracle_prefill, with g [B][Hv][T][dk] (one log-decay per key channel).
 */
int gdn_oracle_kda_prefill(int B, int T, int Hk, int Hv, int dk, int dv, int head_map, double scale,
                           const float *q, const float *k, const float *v,
                           const float *g, const float *beta, const double *s0,
                           const int64_t *pairs, int64_t npairs,
                           double *o, double *s_final, int nthreads) {
    if (check_shape(B, T, Hk, Hv, dk, dv, head_map)) return 1;
    if (!pairs) npairs = (int64_t)B * Hv;
    for (int64_t p = 0; pairs && p < npairs; ++p)
        if (pairs[p] < 0 || pairs[p] >= (int64_t)B * Hv) return 1;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
    for (int64_t p = 0; p < npairs; ++p) {
        int64_t pair = pairs ? pairs[p] : p;
        int b = (int)(pair / Hv), h = (int)(pair % Hv);
        int kh = key_head_of(h, Hk, Hv, head_map);
        double *S = (double *)calloc((size_t)dv * dk, sizeof(double));
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *out = (double *)malloc(sizeof(double) * (size_t)dv);
        double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
        if (!S || !u || !out || !alpha) { bad = 1; free(S); free(u); free(out); free(alpha); continue; }
        if (s0) {
            const double *src = s0 + ((int64_t)b * Hv + h) * dv * dk;
            for (int64_t e = 0; e < (int64_t)dv * dk; ++e) S[e] = src[e];
        }
        for (int t = 0; t < T; ++t) {
            const float *qq = q + (((int64_t)b * Hk + kh) * T + t) * dk;
            const float *kk = k + (((int64_t)b * Hk + kh) * T + t) * dk;
            const float *vv = v + (((int64_t)b * Hv + h) * T + t) * dv;
            int64_t gi = ((int64_t)b * Hv + h) * T + t;
            for (int j = 0; j < dk; ++j) alpha[j] = exp((double)g[gi * dk + j]);
            oracle_kda_step(S, dk, dv, alpha, (double)beta[gi], scale, qq, kk, vv, u, out);
            if (o) memcpy(o + ((int64_t)p * T + t) * dv, out, sizeof(double) * (size_t)dv);
        }
        if (s_final) memcpy(s_final + (int64_t)p * dv * dk, S, sizeof(double) * (size_t)dv * dk);
        free(S); free(u); free(out); free(alpha);
    }
    return bad ? 2 : 0;
}

/*
 * KDA decode step: as gdn_oracle_decode, with g [B][Hv][dk].
 */
int gdn_oracle_kda_decode(int B, int Hk, int Hv, int dk, int dv, int head_map, double scale,
                          const float *q, const float *k, const float *v,
                          const float *g, const float *beta,
                          const int64_t *pairs, int64_t npairs,
                          double *state, double *o, int nthreads) {
    if (check_shape(B, 1, Hk, Hv, dk, dv, head_map)) return 1;
    if (!state || !o) return 1;
    if (!pairs) npairs = (int64_t)B * Hv;
    for (int64_t p = 0; pairs && p < npairs; ++p)
        if (pairs[p] < 0 || pairs[p] >= (int64_t)B * Hv) return 1;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads) reduction(| : bad)
    for (int64_t p = 0; p < npairs; ++p) {
        int64_t pair = pairs ? pairs[p] : p;
        int b = (int)(pair / Hv), h = (int)(pair % Hv);
        int kh = key_head_of(h, Hk, Hv, head_map);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
        if (!u || !alpha) { bad = 1; free(u); free(alpha); continue; }
        const float *qq = q + ((int64_t)b * Hk + kh) * dk;
        const float *kk = k + ((int64_t)b * Hk + kh) * dk;
        const float *vv = v + ((int64_t)b * Hv + h) * dv;
        for (int j = 0; j < dk; ++j) alpha[j] = exp((double)g[pair * dk + j]);
        oracle_kda_step(state + (int64_t)p * dv * dk, dk, dv, alpha, (double)beta[pair], scale,
                        qq, kk, vv, u, o + (int64_t)p * dv);
        free(u); free(alpha);
    }
    return bad ? 2 : 0;
}
