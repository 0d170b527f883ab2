/*
 * Plain fp64 CPU oracle for the Kimi Delta Attention (KDA) forward pass,
 * parallel over (sequence, head) pairs with OpenMP.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path. It shares no code,
 * header or constant with the HIP library.
 *
 * It computes exactly what the numpy oracle (kda_ref.py) computes, token by
 * token, and exists because numpy is too slow at sequence length 8192:
 *
 *   a_t[c]  = max(-exp(A_log[h]) * softplus(g_t[c] + dt_bias[h*K+c]), lb)
 *             (gate inputs named in "Moonshot AI Rilis FlashKDA", API
 *              paragraphs; the pages give no formula, the clamped form is
 *              the reading this oracle takes)
 *   beta_t  = sigmoid(beta logit)          (sigmoid applied inside: same page)
 *   S_t     = (I - beta_t k_t k_t^T) Diag(exp(a_t)) S_{t-1} + beta_t k_t v_t^T
 *             (gated delta rule with channel-wise decay: "Moonshot AI
 *              Open-Sources FlashKDA", section "Why KDA?")
 *   o_t     = scale * S_t^T q_t
 *
 * with the state reset per sequence (cu_seqlens) and optional initial /
 * final states.  Inputs are raw bf16 bit patterns (uint16) and fp32 values;
 * they are widened to fp64 exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_f64(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double softplus64(double x) {
    /* log(1 + e^x), stable for both signs */
    if (x > 0.0) return x + log1p(exp(-x));
    return log1p(exp(x));
}

/*
 * q,k,g: [B*T, H, K] bf16 bits; v: [B*T, H, V]; beta: [B*T, H].
 * cu_seqlens: [num_seqs+1] int32 (B must be 1) or NULL (then N = B, length T
 * each, and num_seqs is ignored).
 * initial_state: [N, H, K, V], dtype 0 = bf16 bits, 1 = fp32; NULL = zeros.
 * heads: the num_sel heads to compute (NULL = all H, num_sel = H).
 * out: [B*T, num_sel, V] fp64; final_state: [N, num_sel, K, V] fp64 or NULL.
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int kda_ref_forward(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const uint16_t *g, const uint16_t *beta,
                    const float *A_log, const float *dt_bias,
                    double lower_bound, double scale,
                    const int32_t *cu_seqlens, int32_t num_seqs,
                    int32_t B, int32_t T,
                    int32_t H, int32_t K, int32_t V,
                    const void *initial_state, int32_t init_dtype,
                    const int32_t *heads, int32_t num_sel,
                    double *out, double *final_state, int32_t num_threads)
{
    if (!q || !k || !v || !g || !beta || !A_log || !out) return -1;
    if (B < 1 || T < 0 || H < 1 || K < 1 || V < 1) return -1;
    if (cu_seqlens && B != 1) return -1;
    int32_t N = cu_seqlens ? num_seqs : B;
    if (N < 0) return -1;
    if (!heads) num_sel = H;
    int64_t tasks = (int64_t)N * num_sel;
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)K * V);
        double *alpha = (double *)malloc(sizeof(double) * (size_t)K);
        double *kk = (double *)malloc(sizeof(double) * (size_t)K);
        double *qq = (double *)malloc(sizeof(double) * (size_t)K);
        double *u = (double *)malloc(sizeof(double) * (size_t)V);
        if (!S || !alpha || !kk || !qq || !u) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t task = 0; task < tasks; task++) {
                int32_t n = (int32_t)(task / num_sel);
                int32_t hs = (int32_t)(task % num_sel);
                int32_t h = heads ? heads[hs] : hs;
                int64_t start, end, row0;
                if (cu_seqlens) { start = cu_seqlens[n]; end = cu_seqlens[n + 1]; row0 = 0; }
                else { start = 0; end = T; row0 = (int64_t)n * T; }
                /* initial state */
                for (int32_t c = 0; c < K; c++)
                    for (int32_t j = 0; j < V; j++) {
                        size_t si = (((size_t)n * H + h) * K + c) * V + j;
                        double s0 = 0.0;
                        if (initial_state)
                            s0 = init_dtype == 0 ? bf16_to_f64(((const uint16_t *)initial_state)[si])
                                                 : (double)((const float *)initial_state)[si];
                        S[(size_t)c * V + j] = s0;
                    }
                double A = exp((double)A_log[h]);
                for (int64_t t = start; t < end; t++) {
                    int64_t row = row0 + t;
                    size_t base_k = ((size_t)row * H + h) * K;
                    size_t base_v = ((size_t)row * H + h) * V;
                    for (int32_t c = 0; c < K; c++) {
                        double x = bf16_to_f64(g[base_k + c]);
                        if (dt_bias) x += (double)dt_bias[(size_t)h * K + c];
                        double a = -A * softplus64(x);
                        if (a < lower_bound) a = lower_bound;
                        alpha[c] = exp(a);
                        kk[c] = bf16_to_f64(k[base_k + c]);
                        qq[c] = bf16_to_f64(q[base_k + c]);
                    }
                    double b = 1.0 / (1.0 + exp(-bf16_to_f64(beta[(size_t)row * H + h])));
                    /* Diag(alpha) S, then S^T k */
                    for (int32_t j = 0; j < V; j++) u[j] = 0.0;
                    for (int32_t c = 0; c < K; c++) {
                        double *Sr = S + (size_t)c * V;
                        double al = alpha[c], kc = kk[c];
                        for (int32_t j = 0; j < V; j++) { Sr[j] *= al; u[j] += kc * Sr[j]; }
                    }
                    /* u = beta (v - S^T k) */
                    for (int32_t j = 0; j < V; j++) u[j] = b * (bf16_to_f64(v[base_v + j]) - u[j]);
                    /* S += k u^T, and o = scale S^T q */
                    double *o = out + ((size_t)row * num_sel + hs) * V;
                    for (int32_t j = 0; j < V; j++) o[j] = 0.0;
                    for (int32_t c = 0; c < K; c++) {
                        double *Sr = S + (size_t)c * V;
                        double kc = kk[c], qc = qq[c];
                        for (int32_t j = 0; j < V; j++) { Sr[j] += kc * u[j]; o[j] += qc * Sr[j]; }
                    }
                    for (int32_t j = 0; j < V; j++) o[j] *= scale;
                }
                if (final_state)
                    memcpy(final_state + ((size_t)n * num_sel + hs) * (size_t)K * V, S,
                           sizeof(double) * (size_t)K * V);
            }
        }
        free(S); free(alpha); free(kk); free(qq); free(u);
    }
    return bad ? -1 : 0;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int kda_ref_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
