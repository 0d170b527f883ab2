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

/*
 * The gradient of kda_ref_forward for the scalar loss
 *     L = <d_out, o> + <d_final, final_state>
 * with respect to every input: the same reverse-mode differentiation of the
 * token recurrence as the numpy gradient oracle (kda_ref_bwd.py, which the
 * CPU tests pin by finite differences), restated in C because numpy is too
 * slow at sequence length 8192.  Per token, with S' = Diag(alpha) S_prev,
 * w = S'^T k, u = beta (v - w), S = S' + k u^T and o = scale S^T q, the
 * gradient dS reaching S is taken back to S_prev through those assignments,
 * last first:
 *     dS += scale q do^T;   dq = scale S do = scale (S' do + k <u, do>)
 *     dk = dS u;            du = dS^T k
 *     dbeta_s = <du, v - w>;  dv = beta du;  dw = -beta du
 *     dS' = dS + k dw^T;    dk += S' dw
 *     dalpha = rowsum(dS' o S_prev);  dS_prev = Diag(alpha) dS'
 * and through the gate a = max(y, lb), y = -exp(A_log) softplus(x),
 * x = g + dt_bias, alpha = e^a (the gradient goes to y where y >= lb):
 *     dy = alpha dalpha where y >= lb, else 0;  dg = dy (-exp(A_log)) sigmoid(x)
 *     ddt_bias = sum of dg over tokens;  dA_log = sum of dy y over tokens, channels
 *     dbeta (of the logit) = dbeta_s beta_s (1 - beta_s).
 * States are recomputed forward from checkpoints kept every `checkpoint`
 * tokens (no arithmetic changes).
 *
 * Arguments as kda_ref_forward, plus d_out [B*T, H, V] bf16 bits and
 * d_final [N, H, K, V] fp32 (NULL = zeros).  Outputs, fp64, for the num_sel
 * selected heads: dq, dk, dg [B*T, num_sel, K]; dv [B*T, num_sel, V];
 * dbeta [B*T, num_sel]; dA_log [num_sel]; ddt_bias [num_sel, K];
 * d_init [N, num_sel, K, V].  Returns 0, or -1 on a bad argument or an
 * allocation failure.
 */
static double sigmoid64(double x) { return 1.0 / (1.0 + exp(-x)); }

/* one token of the forward recurrence on S (K x V, in place): S <- S_t */
static void token_step(double *S, const double *alpha, const double *kk, const double *vv,
                       double b, double *u, int32_t K, int32_t V) {
    for (int32_t j = 0; j < V; j++) u[j] = 0.0;
    for (int32_t c = 0; c < K; c++) {
        double *Sr = S + (size_t)c * V;
        for (int32_t j = 0; j < V; j++) { Sr[j] *= alpha[c]; u[j] += kk[c] * Sr[j]; }
    }
    for (int32_t j = 0; j < V; j++) u[j] = b * (vv[j] - u[j]);
    for (int32_t c = 0; c < K; c++) {
        double *Sr = S + (size_t)c * V;
        for (int32_t j = 0; j < V; j++) Sr[j] += kk[c] * u[j];
    }
}

int kda_ref_backward(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const uint16_t *g, const uint16_t *beta,
                     const float *A_log, const float *dt_bias,
                     double lower_bound, double scale,
                     const int32_t *cu_seqlens, int32_t num_seqs,
                     int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                     const void *initial_state, int32_t init_dtype,
                     const uint16_t *d_out, const float *d_final,
                     const int32_t *heads, int32_t num_sel, int32_t checkpoint,
                     double *dq, double *dk, double *dv, double *dg, double *dbeta,
                     double *dA_log, double *ddt_bias, double *d_init, int32_t num_threads)
{
    if (!q || !k || !v || !g || !beta || !A_log || !d_out) return -1;
    if (!dq || !dk || !dv || !dg || !dbeta || !dA_log || !ddt_bias || !d_init) return -1;
    if (B < 1 || T < 0 || H < 1 || K < 1 || V < 1 || checkpoint < 1) return -1;
    if (cu_seqlens && B != 1) return -1;
    int32_t N = cu_seqlens ? num_seqs : B;
    if (N < 0) return -1;
    if (!heads) num_sel = H;
    const int64_t tasks = (int64_t)N * num_sel;
    const size_t KV = (size_t)K * V;
    /* per (sequence, head) partial sums of dA_log and ddt_bias, summed over
       the sequences after the parallel region */
    double *pa = (double *)calloc((size_t)(tasks > 0 ? tasks : 1), sizeof(double));
    double *pd = (double *)calloc((size_t)(tasks > 0 ? tasks : 1) * K, sizeof(double));
    if (!pa || !pd) { free(pa); free(pd); return -1; }
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * KV);
        double *Sp = (double *)malloc(sizeof(double) * KV);
        double *dS = (double *)malloc(sizeof(double) * KV);
        double *seg = (double *)malloc(sizeof(double) * KV * (size_t)checkpoint);
        double *kvec = (double *)malloc(sizeof(double) * (size_t)K * 7);
        double *vvec = (double *)malloc(sizeof(double) * (size_t)V * 6);
        if (!S || !Sp || !dS || !seg || !kvec || !vvec) {
#pragma omp atomic write
            bad = 1;
        } else {
            double *alpha = kvec, *y = kvec + K, *x = kvec + 2 * K, *kk = kvec + 3 * K;
            double *qq = kvec + 4 * K, *dkv = kvec + 5 * K, *dal = kvec + 6 * K;
            double *vv = vvec, *dov = vvec + V, *w = vvec + 2 * V, *u = vvec + 3 * V;
            double *du = vvec + 4 * V, *dw = vvec + 5 * V;
#pragma omp for schedule(dynamic, 1)
            for (int64_t task = 0; task < tasks; task++) {
                const int32_t n = (int32_t)(task / num_sel);
                const int32_t hs = (int32_t)(task % num_sel);
                const int32_t h = heads ? heads[hs] : hs;
                int64_t start, end, row0;
                if (cu_seqlens) { start = cu_seqlens[n]; end = cu_seqlens[n + 1]; row0 = 0; }
                else { start = 0; end = T; row0 = (int64_t)n * T; }
                const double A = exp((double)A_log[h]);
                /* gate, beta and the token's vectors of token t of this head */
#define LOAD_TOKEN(t_)                                                                     \
                do {                                                                       \
                    const int64_t row_ = row0 + (t_);                                      \
                    const size_t bk_ = ((size_t)row_ * H + h) * K;                         \
                    const size_t bv_ = ((size_t)row_ * H + h) * V;                         \
                    for (int32_t c = 0; c < K; c++) {                                      \
                        x[c] = bf16_to_f64(g[bk_ + c]) +                                   \
                               (dt_bias ? (double)dt_bias[(size_t)h * K + c] : 0.0);       \
                        y[c] = -A * softplus64(x[c]);                                      \
                        alpha[c] = exp(y[c] < lower_bound ? lower_bound : y[c]);           \
                        kk[c] = bf16_to_f64(k[bk_ + c]);                                   \
                        qq[c] = bf16_to_f64(q[bk_ + c]);                                   \
                    }                                                                      \
                    for (int32_t j = 0; j < V; j++) vv[j] = bf16_to_f64(v[bv_ + j]);        \
                    bt = sigmoid64(bf16_to_f64(beta[(size_t)row_ * H + h]));               \
                } while (0)
                double bt = 0.0;
                for (int32_t c = 0; c < K; c++)
                    for (int32_t j = 0; j < V; j++) {
                        const size_t si = (((size_t)n * H + h) * K + c) * V + j;
                        double s0 = 0.0;
                        if (initial_state)
                            s0 = init_dtype == 0 ? bf16_to_f64(((const uint16_t *)initial_state)[si])
                                                 : (double)((const float *)initial_state)[si];
                        S[(size_t)c * V + j] = s0;
                    }
                const int64_t L = end - start;
                const int64_t nck = (L + checkpoint - 1) / checkpoint;
                double *ckpt = (double *)malloc(sizeof(double) * KV * (size_t)(nck > 0 ? nck : 1));
                if (!ckpt) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                /* forward: the state before every checkpoint-th token */
                for (int64_t t = start; t < end; t++) {
                    if ((t - start) % checkpoint == 0)
                        memcpy(ckpt + KV * (size_t)((t - start) / checkpoint), S, sizeof(double) * KV);
                    LOAD_TOKEN(t);
                    token_step(S, alpha, kk, vv, bt, u, K, V);
                }
                for (size_t i = 0; i < KV; i++)
                    dS[i] = d_final ? (double)d_final[(((size_t)n * H + h) * KV) + i] : 0.0;
                for (int64_t sgi = nck - 1; sgi >= 0; sgi--) {
                    const int64_t s0 = start + sgi * checkpoint;
                    const int64_t s1 = s0 + checkpoint < end ? s0 + checkpoint : end;
                    /* seg[i]: the state before token s0 + i */
                    memcpy(seg, ckpt + KV * (size_t)sgi, sizeof(double) * KV);
                    for (int64_t t = s0; t + 1 < s1; t++) {
                        double *nx = seg + KV * (size_t)(t - s0 + 1);
                        memcpy(nx, seg + KV * (size_t)(t - s0), sizeof(double) * KV);
                        LOAD_TOKEN(t);
                        token_step(nx, alpha, kk, vv, bt, u, K, V);
                    }
                    for (int64_t t = s1 - 1; t >= s0; t--) {
                        const double *Sprev = seg + KV * (size_t)(t - s0);
                        LOAD_TOKEN(t);
                        const int64_t row = row0 + t;
                        const size_t bo = ((size_t)row * H + h) * V;
                        for (int32_t j = 0; j < V; j++) { dov[j] = bf16_to_f64(d_out[bo + j]); w[j] = 0.0; }
                        for (int32_t c = 0; c < K; c++)
                            for (int32_t j = 0; j < V; j++) {
                                Sp[(size_t)c * V + j] = alpha[c] * Sprev[(size_t)c * V + j];
                                w[j] += kk[c] * Sp[(size_t)c * V + j];
                            }
                        double ud = 0.0;
                        for (int32_t j = 0; j < V; j++) { u[j] = bt * (vv[j] - w[j]); ud += u[j] * dov[j]; }
                        const size_t ok = ((size_t)row * num_sel + hs) * K;
                        const size_t ov = ((size_t)row * num_sel + hs) * V;
                        for (int32_t c = 0; c < K; c++) {
                            double sdo = 0.0;
                            for (int32_t j = 0; j < V; j++) sdo += Sp[(size_t)c * V + j] * dov[j];
                            dq[ok + c] = scale * (sdo + kk[c] * ud);
                        }
                        for (int32_t j = 0; j < V; j++) du[j] = 0.0;
                        for (int32_t c = 0; c < K; c++) {
                            double *dr = dS + (size_t)c * V;
                            double acc = 0.0;
                            for (int32_t j = 0; j < V; j++) {
                                dr[j] += scale * qq[c] * dov[j];
                                acc += dr[j] * u[j];
                                du[j] += dr[j] * kk[c];
                            }
                            dkv[c] = acc;
                        }
                        double dbs = 0.0;
                        for (int32_t j = 0; j < V; j++) {
                            dbs += du[j] * (vv[j] - w[j]);
                            dv[ov + j] = bt * du[j];
                            dw[j] = -bt * du[j];
                        }
                        for (int32_t c = 0; c < K; c++) {
                            double *dr = dS + (size_t)c * V;
                            const double *sp = Sp + (size_t)c * V, *pr = Sprev + (size_t)c * V;
                            double acc = 0.0, da = 0.0;
                            for (int32_t j = 0; j < V; j++) {
                                dr[j] += kk[c] * dw[j];
                                acc += sp[j] * dw[j];
                                da += dr[j] * pr[j];
                            }
                            dk[ok + c] = dkv[c] + acc;
                            dal[c] = da;
                            for (int32_t j = 0; j < V; j++) dr[j] *= alpha[c];
                        }
                        for (int32_t c = 0; c < K; c++) {
                            const double dy = y[c] >= lower_bound ? alpha[c] * dal[c] : 0.0;
                            const double dx = dy * (-A) * sigmoid64(x[c]);
                            dg[ok + c] = dx;
                            pd[(size_t)task * K + c] += dx;
                            pa[task] += dy * y[c];
                        }
                        dbeta[(size_t)row * num_sel + hs] = dbs * bt * (1.0 - bt);
                    }
                }
#undef LOAD_TOKEN
                memcpy(d_init + ((size_t)n * num_sel + hs) * KV, dS, sizeof(double) * KV);
                free(ckpt);
            }
        }
        free(S); free(Sp); free(dS); free(seg); free(kvec); free(vvec);
    }
    if (!bad) {
        for (int32_t hs = 0; hs < num_sel; hs++) {
            double a = 0.0;
            for (int32_t n = 0; n < N; n++) a += pa[(size_t)n * num_sel + hs];
            dA_log[hs] = a;
            for (int32_t c = 0; c < K; c++) {
                double d = 0.0;
                for (int32_t n = 0; n < N; n++) d += pd[((size_t)n * num_sel + hs) * K + c];
                ddt_bias[(size_t)hs * K + c] = d;
            }
        }
    }
    free(pa); free(pd);
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
