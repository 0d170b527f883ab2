// Backward pass: the gradient of the chunked forward with respect to every
// input.  The pages ship the forward only and leave training to another
// backend ("Moonshot AI Open-Sources FlashKDA", section "Limitations before
// you integrate"), so this is the derivative of the forward this library
// computes, taken through the same chunkwise form (kda_device.h):
//
//   X  = V - Kt S0,   O = scale (Qt S0 + M X),   S1 = Gam S0 + Wm^T X
//   Kt = k e^G, Qt = q e^G, Kb = k e^-G, Gam = diag(e^{G_last})
//   T  = (I + diag(beta) strict_lower(Kt Kb^T))^-1,  P = T diag(beta)
//   Aqk = lower_incl(Qt Kb^T),  M = Aqk P,  Wm = P^T Kb Gam
//
// Given dO and the gradient reaching each chunk's end state dS1, the chain
// rule through those assignments gives
//
//   dX  = scale M^T dO + Wm dS1              dV = dX
//   dS0 = Gam dS1 + scale Qt^T dO - Kt^T dX   (the reverse recurrence)
//   dQt = scale dO S0^T,  dKt = -dX S0^T,  dWm = X dS1^T,  dM = scale dO X^T,
//   dGam = diag(dS1 S0^T)
//
// and, inside the chunk, through M, Wm, P, T and the two Gram products down
// to dq, dk, dbeta and the in-chunk cumulative decay G, whose reverse
// cumulative sum is the gradient of the per-token log-decay; the gate
// a = max(-exp(A_log) softplus(g + dt_bias), lower_bound) then yields dg,
// dA_log and ddt_bias (no gradient through the clamped branch).
//
// Five launches, all fp32 arithmetic:
//   prep    (chunk slot, head)  the chunk factors Kt, Qt, Wm, M, Gam -> workspace
//   states  (sequence, head, 32-column part)  forward scan storing every
//           chunk's start state S0
//   dstates (sequence, head, 32-column part)  reverse scan of dS, storing
//           every chunk's dS1, writing dv and the initial-state gradient
//   chunk   (chunk slot, head)  the products with S0 / dS1 and the in-chunk
//           backward: dq, dk, dg, dbeta, per-chunk dA_log / ddt_bias sums
//   reduce  (head)  sums the per-chunk parameter gradients in slot order
// Every sum runs in a fixed order, so results are bitwise reproducible.
#include <math.h>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int BT = 256;               // threads per workgroup
constexpr int RS = HD + 4;            // padded LDS row stride (floats)
constexpr int SP = CS + 1;            // padded stride of 16 x 16 tiles
constexpr int CWB = 32;               // state columns per scan workgroup
constexpr int NPART = HD / CWB;
constexpr int NRG = BT / CWB;         // row groups of 16 state rows
static_assert(NRG * 16 == HD, "row groups cover the state rows");

// Chunk-factor record, fp32, per (chunk slot, head).
constexpr int BR_KT = 0;
constexpr int BR_QT = CS * HD;
constexpr int BR_WM = 2 * CS * HD;
constexpr int BR_M = 3 * CS * HD;
constexpr int BR_GAM = 3 * CS * HD + CS * CS;
constexpr int BR_FLOATS = BR_GAM + HD;

__device__ __forceinline__ float softplus_f(float x) {
    return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

// Token range of chunk slot `slot`: returns its token count (0 for a gap
// slot) and the first token row in t0.
__device__ int slot_chunk(const int32_t *cu, int N, int T, int64_t slot, int64_t &t0) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seq_slot0(cu, mid, T) <= slot) lo = mid; else hi = mid - 1;
    }
    int64_t start, end;
    seq_range(cu, lo, T, start, end);
    t0 = start + (slot - seq_slot0(cu, lo, T)) * CS;
    return t0 >= end ? 0 : (int)min((int64_t)CS, end - t0);
}

// ---------------------------------------------------------------------------
// Chunk factors of one (chunk, head) in LDS.  Rows from `len` on are padding:
// zero k, q and beta and a zero log-decay, which makes every factor row and
// column they touch zero (and e^{G_last} that of the last real token).
// ---------------------------------------------------------------------------
struct Factors {
    float kt[CS][RS], qt[CS][RS], kb[CS][RS], e[CS][RS], wm[CS][RS];
    float A[CS][SP], aqk[CS][SP], T[CS][SP], P[CS][SP], M[CS][SP];
    float beta[CS], gam[HD], dtb[HD];
};

__device__ void chunk_factors(Factors &L, const uint16_t *__restrict__ q,
                              const uint16_t *__restrict__ k, const uint16_t *__restrict__ g,
                              const uint16_t *__restrict__ bl, float Aexp,
                              const float *__restrict__ dt_bias, float lb, int64_t t0, int len,
                              int H, int h) {
    const int tid = threadIdx.x;
    if (tid < HD) {
        // one channel per thread: gate, in-chunk cumulative log-decay G
        // (natural log) and the scaled rows
        const int c = tid;
        const float dtb = dt_bias ? dt_bias[(size_t)h * HD + c] : 0.f;
        L.dtb[c] = dtb;
        float G = 0.f;
#pragma unroll
        for (int r = 0; r < CS; ++r) {
            float kv = 0.f, qv = 0.f;
            if (r < len) {
                const size_t off = ((size_t)(t0 + r) * H + h) * HD + c;
                G += fmaxf(-Aexp * softplus_f(bf16f(g[off]) + dtb), lb);
                kv = bf16f(k[off]);
                qv = bf16f(q[off]);
            }
            const float e = expf(G);
            L.e[r][c] = e;
            L.kt[r][c] = kv * e;
            L.qt[r][c] = qv * e;
            L.kb[r][c] = kv * expf(-G);
        }
        L.gam[c] = L.e[CS - 1][c];
    } else if (tid < HD + CS) {
        const int r = tid - HD;
        L.beta[r] = r < len ? sigmoid_f(bf16f(bl[(size_t)(t0 + r) * H + h])) : 0.f;
    }
    __syncthreads();
    {
        // A = strict_lower(Kt Kb^T), Aqk = lower_incl(Qt Kb^T)
        const int r = tid >> 4, i = tid & 15;
        float a = 0.f, aq = 0.f;
        for (int c = 0; c < HD; c += 4) {
            const float4 b4 = *(const float4 *)&L.kb[i][c];
            const float4 t4 = *(const float4 *)&L.kt[r][c];
            const float4 q4 = *(const float4 *)&L.qt[r][c];
            a += t4.x * b4.x + t4.y * b4.y + t4.z * b4.z + t4.w * b4.w;
            aq += q4.x * b4.x + q4.y * b4.y + q4.z * b4.z + q4.w * b4.w;
        }
        L.A[r][i] = i < r ? a : 0.f;
        L.aqk[r][i] = i <= r ? aq : 0.f;
    }
    __syncthreads();
    if (tid < CS) {
        // column i of T = (I + diag(beta) A)^-1 by forward substitution
        const int i = tid;
        for (int r = 0; r < CS; ++r) {
            float acc = r == i ? 1.f : 0.f;
            for (int s = i; s < r; ++s) acc -= L.beta[r] * L.A[r][s] * L.T[s][i];
            L.T[r][i] = acc;
        }
    }
    __syncthreads();
    {
        const int r = tid >> 4, i = tid & 15;
        L.P[r][i] = L.T[r][i] * L.beta[i];
    }
    __syncthreads();
    {
        const int r = tid >> 4, i = tid & 15;
        float m = 0.f;
        for (int s = 0; s < CS; ++s) m += L.aqk[r][s] * L.P[s][i];
        L.M[r][i] = m;
        const int c = tid & (HD - 1), i0 = tid >> 7;
        for (int mm = 0; mm < CS / 2; ++mm) {
            const int ii = i0 + 2 * mm;
            float w = 0.f;
            for (int s = 0; s < CS; ++s) w += L.P[s][ii] * L.kb[s][c];
            L.wm[ii][c] = w * L.gam[c];
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// prep: chunk factors -> workspace record (fp32, BR_FLOATS per slot x head)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(BT) void bwd_prep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ g, const uint16_t *__restrict__ beta,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float lb,
    const int32_t *__restrict__ cu, int N, int T, int H, float *__restrict__ brec)
{
    __shared__ __attribute__((aligned(16))) Factors L;
    const int64_t slot = blockIdx.x / (unsigned)H;
    const int h = (int)(blockIdx.x % (unsigned)H);
    int64_t t0;
    const int len = slot_chunk(cu, N, T, slot, t0);
    if (len == 0) return;                                   // gap slot
    chunk_factors(L, q, k, g, beta, expf(A_log[h]), dt_bias, lb, t0, len, H, h);
    float *rec = brec + ((size_t)slot * H + h) * BR_FLOATS;
    const int tid = threadIdx.x;
    for (int idx = tid; idx < CS * HD; idx += BT) {
        const int r = idx / HD, c = idx % HD;
        rec[BR_KT + idx] = L.kt[r][c];
        rec[BR_QT + idx] = L.qt[r][c];
        rec[BR_WM + idx] = L.wm[r][c];
    }
    rec[BR_M + tid] = L.M[tid >> 4][tid & 15];
    if (tid < HD) rec[BR_GAM + tid] = L.gam[tid];
}

// ---------------------------------------------------------------------------
// states: forward scan per (sequence, head, 32-column part) that stores each
// chunk's start state S0 (fp32 [slot][head][K][V]).  Thread t holds column
// t % 32 of the part and rows 16 (t / 32) .. +15 of the state.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(BT) void bwd_states_kernel(
    const uint16_t *__restrict__ v, const float *__restrict__ brec,
    const int32_t *__restrict__ cu, int N, int T, int H,
    const void *__restrict__ init, int init_fp32, float *__restrict__ st0)
{
    __shared__ float kt[CS][HD], wm[CS][HD], gam[HD];
    __shared__ float vv[CS][CWB], xs[CS][CWB], xp[NRG][CS][CWB];
    const int unit = blockIdx.x;
    const int part = unit % NPART, nh = unit / NPART;
    const int h = nh % H, n = nh / H;
    const int tid = threadIdx.x, j = tid % CWB, rg = tid / CWB;
    const int col = part * CWB + j;
    const size_t sbase = ((size_t)n * H + h) * HD * HD;

    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const size_t idx = sbase + (size_t)(rg * 16 + i) * HD + col;
        s[i] = !init ? 0.f : init_fp32 ? ((const float *)init)[idx]
                                       : bf16f(((const uint16_t *)init)[idx]);
    }
    int64_t start, end;
    seq_range(cu, n, T, start, end);
    const int nch = (int)((end - start + CS - 1) / CS);
    const int64_t slot0 = seq_slot0(cu, n, T);
    for (int ci = 0; ci < nch; ++ci) {
        const int64_t slot = slot0 + ci;
        const float *rec = brec + ((size_t)slot * H + h) * BR_FLOATS;
        float *dst = st0 + ((size_t)slot * H + h) * HD * HD;
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(size_t)(rg * 16 + i) * HD + col] = s[i];
        const int64_t t0 = start + (int64_t)ci * CS;
        const int len = (int)min((int64_t)CS, end - t0);
        __syncthreads();                                    // last chunk's readers are done
        for (int idx = tid; idx < CS * HD; idx += BT) {
            kt[idx / HD][idx % HD] = rec[BR_KT + idx];
            wm[idx / HD][idx % HD] = rec[BR_WM + idx];
        }
        if (tid < HD) gam[tid] = rec[BR_GAM + tid];
        for (int idx = tid; idx < CS * CWB; idx += BT) {
            const int r = idx / CWB, jj = idx % CWB;
            vv[r][jj] = r < len ? bf16f(v[((size_t)(t0 + r) * H + h) * HD + part * CWB + jj]) : 0.f;
        }
        __syncthreads();
        // X = V - Kt S0: partial sums over this thread's 16 rows
        for (int r = 0; r < CS; ++r) {
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) p += kt[r][rg * 16 + i] * s[i];
            xp[rg][r][j] = p;
        }
        __syncthreads();
        for (int m = 0; m < 2; ++m) {
            const int r = 2 * rg + m;
            float x = vv[r][j];
            for (int gq = 0; gq < NRG; ++gq) x -= xp[gq][r][j];
            xs[r][j] = x;
        }
        __syncthreads();
        // S1 = Gam S0 + Wm^T X
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int c = rg * 16 + i;
            float acc = gam[c] * s[i];
            for (int r = 0; r < CS; ++r) acc += wm[r][c] * xs[r][j];
            s[i] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// dstates: reverse scan per (sequence, head, 32-column part) of the state
// gradient.  Stores dS1 of every chunk (fp32 [slot][head][K][V]), writes dv
// and, at the sequence start, the initial-state gradient.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(BT) void bwd_dstates_kernel(
    const uint16_t *__restrict__ dout, const float *__restrict__ brec,
    const int32_t *__restrict__ cu, int N, int T, int H, float scale,
    const float *__restrict__ dfin, float *__restrict__ dst1, uint16_t *__restrict__ dv,
    float *__restrict__ dinit)
{
    __shared__ float kt[CS][HD], qt[CS][HD], wm[CS][HD], gam[HD], Ml[CS][SP];
    __shared__ float dol[CS][CWB], dxs[CS][CWB], xp[NRG][CS][CWB];
    const int unit = blockIdx.x;
    const int part = unit % NPART, nh = unit / NPART;
    const int h = nh % H, n = nh / H;
    const int tid = threadIdx.x, j = tid % CWB, rg = tid / CWB;
    const int col = part * CWB + j;
    const size_t sbase = ((size_t)n * H + h) * HD * HD;

    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        ds[i] = dfin ? dfin[sbase + (size_t)(rg * 16 + i) * HD + col] : 0.f;
    int64_t start, end;
    seq_range(cu, n, T, start, end);
    const int nch = (int)((end - start + CS - 1) / CS);
    const int64_t slot0 = seq_slot0(cu, n, T);
    for (int ci = nch - 1; ci >= 0; --ci) {
        const int64_t slot = slot0 + ci;
        const float *rec = brec + ((size_t)slot * H + h) * BR_FLOATS;
        float *dst = dst1 + ((size_t)slot * H + h) * HD * HD;
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(size_t)(rg * 16 + i) * HD + col] = ds[i];
        const int64_t t0 = start + (int64_t)ci * CS;
        const int len = (int)min((int64_t)CS, end - t0);
        __syncthreads();
        for (int idx = tid; idx < CS * HD; idx += BT) {
            kt[idx / HD][idx % HD] = rec[BR_KT + idx];
            qt[idx / HD][idx % HD] = rec[BR_QT + idx];
            wm[idx / HD][idx % HD] = rec[BR_WM + idx];
        }
        Ml[tid >> 4][tid & 15] = rec[BR_M + tid];
        if (tid < HD) gam[tid] = rec[BR_GAM + tid];
        for (int idx = tid; idx < CS * CWB; idx += BT) {
            const int r = idx / CWB, jj = idx % CWB;
            dol[r][jj] = r < len
                ? scale * bf16f(dout[((size_t)(t0 + r) * H + h) * HD + part * CWB + jj]) : 0.f;
        }
        __syncthreads();
        // dX = scale M^T dO + Wm dS1: partial sums of Wm dS1 over this thread's rows
        for (int r = 0; r < CS; ++r) {
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) p += wm[r][rg * 16 + i] * ds[i];
            xp[rg][r][j] = p;
        }
        __syncthreads();
        for (int m = 0; m < 2; ++m) {
            const int r = 2 * rg + m;
            float x = 0.f;
            for (int sr = 0; sr < CS; ++sr) x += Ml[sr][r] * dol[sr][j];
            for (int gq = 0; gq < NRG; ++gq) x += xp[gq][r][j];
            dxs[r][j] = x;
            if (r < len) dv[((size_t)(t0 + r) * H + h) * HD + col] = tobf16(x);
        }
        __syncthreads();
        // dS0 = Gam dS1 + scale Qt^T dO - Kt^T dX
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int c = rg * 16 + i;
            float acc = gam[c] * ds[i];
            for (int r = 0; r < CS; ++r) acc += qt[r][c] * dol[r][j] - kt[r][c] * dxs[r][j];
            ds[i] = acc;
        }
    }
    if (dinit) {
#pragma unroll
        for (int i = 0; i < 16; ++i) dinit[sbase + (size_t)(rg * 16 + i) * HD + col] = ds[i];
    }
}

// ---------------------------------------------------------------------------
// chunk: per (chunk slot, head), everything that needs S0 and dS1 of the
// chunk, then the in-chunk backward down to the inputs.
// ---------------------------------------------------------------------------
struct ChunkLds {
    Factors f;
    float dol[CS][RS], vl[CS][RS];        // scale * dO, v
    float s0b[CS][RS], ds1b[CS][RS];      // 16-channel row blocks of S0 and dS1
    float x[CS][RS], dx[CS][RS];
    float dqt[CS][RS], dkt[CS][RS], dwm[CS][RS];
    float dM[CS][SP], dAqk[CS][SP], dP[CS][SP], Y[CS][SP], dL[CS][SP], dA[CS][SP];
    float dgam[HD], dgam2[2][HD], red[BT / 64];
};

__device__ __forceinline__ void load_block(float (&dst)[CS][RS], const float *__restrict__ src) {
    // 16 rows x 128 floats, contiguous in global memory
    const int tid = threadIdx.x;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int idx = 4 * (tid + m * BT);
        *(float4 *)&dst[idx / HD][idx % HD] = *(const float4 *)&src[idx];
    }
}

__global__ __launch_bounds__(BT) void bwd_chunk_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ g,
    const uint16_t *__restrict__ beta, const float *__restrict__ A_log,
    const float *__restrict__ dt_bias, float lb, float scale, const uint16_t *__restrict__ dout,
    const int32_t *__restrict__ cu, int N, int T, int H,
    const float *__restrict__ st0, const float *__restrict__ dst1,
    uint16_t *__restrict__ dq, uint16_t *__restrict__ dk, uint16_t *__restrict__ dg,
    uint16_t *__restrict__ dbeta, float *__restrict__ part_alog, float *__restrict__ part_dtb)
{
    __shared__ __attribute__((aligned(16))) ChunkLds L;
    Factors &F = L.f;
    const int64_t slot = blockIdx.x / (unsigned)H;
    const int h = (int)(blockIdx.x % (unsigned)H);
    const int tid = threadIdx.x;
    const size_t sh = (size_t)slot * H + h;
    int64_t t0;
    const int len = slot_chunk(cu, N, T, slot, t0);
    if (len == 0) {                                         // gap slot: zero partial sums
        if (tid < HD) part_dtb[sh * HD + tid] = 0.f;
        if (tid == 0) part_alog[sh] = 0.f;
        return;
    }
    const float Aexp = expf(A_log[h]);
    chunk_factors(F, q, k, g, beta, Aexp, dt_bias, lb, t0, len, H, h);

    for (int idx = tid; idx < CS * HD; idx += BT) {
        const int r = idx / HD, c = idx % HD;
        const size_t off = ((size_t)(t0 + r) * H + h) * HD + c;
        L.dol[r][c] = r < len ? scale * bf16f(dout[off]) : 0.f;
        L.vl[r][c] = r < len ? bf16f(v[off]) : 0.f;
    }
    const float *S0 = st0 + sh * HD * HD;
    const float *DS = dst1 + sh * HD * HD;

    // pass 1 over 16-channel blocks: X, dX (accumulated), dQt, dGam
    const int r_ = tid >> 4, lo = tid & 15, j0 = lo * 8;
    float xa[8], dxa[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) xa[m] = dxa[m] = 0.f;
    for (int cb = 0; cb < HD / 16; ++cb) {
        __syncthreads();
        load_block(L.s0b, S0 + (size_t)cb * 16 * HD);
        load_block(L.ds1b, DS + (size_t)cb * 16 * HD);
        __syncthreads();
        for (int cc = 0; cc < 16; ++cc) {
            const int c = cb * 16 + cc;
            const float ktv = F.kt[r_][c], wmv = F.wm[r_][c];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                xa[m] -= ktv * L.s0b[cc][j0 + m];
                dxa[m] += wmv * L.ds1b[cc][j0 + m];
            }
        }
        {
            float acc = 0.f;
            for (int jj = 0; jj < HD; jj += 4) {
                const float4 a4 = *(const float4 *)&L.dol[r_][jj];
                const float4 b4 = *(const float4 *)&L.s0b[lo][jj];
                acc += a4.x * b4.x + a4.y * b4.y + a4.z * b4.z + a4.w * b4.w;
            }
            L.dqt[r_][cb * 16 + lo] = acc;
        }
        {
            // dGam[c] = sum_j dS1[c][j] S0[c][j]: 16 lanes per channel, 8 columns each
            const int cc = tid >> 4;
            float p = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) p += L.ds1b[cc][j0 + m] * L.s0b[cc][j0 + m];
            p += __shfl_xor(p, 8, 16);
            p += __shfl_xor(p, 4, 16);
            p += __shfl_xor(p, 2, 16);
            p += __shfl_xor(p, 1, 16);
            if (lo == 0) L.dgam[cb * 16 + cc] = p;
        }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        float d = dxa[m];
        for (int sr = 0; sr < CS; ++sr) d += F.M[sr][r_] * L.dol[sr][j0 + m];
        L.x[r_][j0 + m] = xa[m] + L.vl[r_][j0 + m];
        L.dx[r_][j0 + m] = d;
    }
    // pass 2 over 16-channel blocks: dKt = -dX S0^T, dWm = X dS1^T
    for (int cb = 0; cb < HD / 16; ++cb) {
        __syncthreads();
        load_block(L.s0b, S0 + (size_t)cb * 16 * HD);
        load_block(L.ds1b, DS + (size_t)cb * 16 * HD);
        __syncthreads();
        float a = 0.f, b = 0.f;
        for (int jj = 0; jj < HD; jj += 4) {
            const float4 dx4 = *(const float4 *)&L.dx[r_][jj];
            const float4 x4 = *(const float4 *)&L.x[r_][jj];
            const float4 s4 = *(const float4 *)&L.s0b[lo][jj];
            const float4 d4 = *(const float4 *)&L.ds1b[lo][jj];
            a += dx4.x * s4.x + dx4.y * s4.y + dx4.z * s4.z + dx4.w * s4.w;
            b += x4.x * d4.x + x4.y * d4.y + x4.z * d4.z + x4.w * d4.w;
        }
        L.dkt[r_][cb * 16 + lo] = -a;
        L.dwm[r_][cb * 16 + lo] = b;
    }
    {
        // dM = scale dO X^T
        float acc = 0.f;
        for (int jj = 0; jj < HD; jj += 4) {
            const float4 a4 = *(const float4 *)&L.dol[r_][jj];
            const float4 b4 = *(const float4 *)&L.x[lo][jj];
            acc += a4.x * b4.x + a4.y * b4.y + a4.z * b4.z + a4.w * b4.w;
        }
        L.dM[r_][lo] = acc;
    }
    __syncthreads();
    {
        // M = Aqk P:  dAqk = dM P^T (lower incl.),  dP = Aqk^T dM
        // Wm = P^T Kb Gam:  dP += Kb Gam dWm^T
        const int r = r_, i = lo;
        float a = 0.f, p = 0.f;
        for (int s = 0; s < CS; ++s) {
            a += L.dM[r][s] * F.P[i][s];
            p += F.aqk[s][r] * L.dM[s][i];
        }
        for (int c = 0; c < HD; ++c) p += F.kb[r][c] * F.gam[c] * L.dwm[i][c];
        L.dAqk[r][i] = i <= r ? a : 0.f;
        L.dP[r][i] = p;
    }
    __syncthreads();
    {
        // P = T diag(beta):  dT = dP diag(beta);  Y = dT T^T
        const int a = r_, s = lo;
        float y = 0.f;
        for (int b = 0; b < CS; ++b) y += L.dP[a][b] * F.beta[b] * F.T[s][b];
        L.Y[a][s] = y;
    }
    __syncthreads();
    {
        // T = (I + L)^-1:  dL = -T^T dT T^T (strictly lower);  L = diag(beta) A
        const int r = r_, s = lo;
        float d = 0.f;
        for (int a = 0; a < CS; ++a) d += F.T[a][r] * L.Y[a][s];
        d = s < r ? -d : 0.f;
        L.dL[r][s] = d;
        L.dA[r][s] = F.beta[r] * d;
    }
    __syncthreads();
    {
        // per (token row r, channel c): the gradients of Qt, Kt, Kb, then q, k, G
        const int c = tid & (HD - 1), rh = tid >> 7;
        float dgk = 0.f;
#pragma unroll 1
        for (int mm = 0; mm < CS / 2; ++mm) {
            const int r = rh + 2 * mm;
            float dQt = L.dqt[r][c], dKt = L.dkt[r][c], dKbG = 0.f, dKb = 0.f;
            for (int s = 0; s < CS; ++s) {
                const float kbs = F.kb[s][c];
                dQt += L.dAqk[r][s] * kbs;                  // zero for s > r
                dKt += L.dA[r][s] * kbs;                    // zero for s >= r
                dKbG += F.P[r][s] * L.dwm[s][c];
                dKb += L.dAqk[s][r] * F.qt[s][c] + L.dA[s][r] * F.kt[s][c];
            }
            dKb += F.gam[c] * dKbG;
            dgk += dKbG * F.kb[r][c];
            const float e = F.e[r][c];
            if (r < len) {
                const size_t off = ((size_t)(t0 + r) * H + h) * HD + c;
                dq[off] = tobf16(dQt * e);
                dk[off] = tobf16(dKt * e + dKb / e);
            }
            // dG (natural log) of this row; stored over dqt, read only by this thread
            L.dqt[r][c] = dKt * F.kt[r][c] + dQt * F.qt[r][c] - dKb * F.kb[r][c];
        }
        L.dgam2[rh][c] = dgk;
    }
    __syncthreads();
    if (tid < HD) {
        // reverse cumulative sum of dG is the gradient of the per-token log-decay;
        // then the gate chain
        const int c = tid;
        const float dgam = L.dgam[c] + L.dgam2[0][c] + L.dgam2[1][c];
        float acc = dgam * F.gam[c];
        float pdtb = 0.f, pa = 0.f;
        for (int s = CS - 1; s >= 0; --s) {
            acc += L.dqt[s][c];
            if (s < len) {
                const size_t off = ((size_t)(t0 + s) * H + h) * HD + c;
                const float x = bf16f(g[off]) + F.dtb[c];
                const float y = -Aexp * softplus_f(x);
                const float dy = y >= lb ? acc : 0.f;
                const float dx = -dy * Aexp * sigmoid_f(x);
                dg[off] = tobf16(dx);
                pdtb += dx;
                pa += dy * y;
            }
        }
        part_dtb[sh * HD + c] = pdtb;
        // sum pa over the 128 channel threads (two waves) in a fixed order
        for (int o = 32; o >= 1; o >>= 1) pa += __shfl_xor(pa, o, 64);
        if ((tid & 63) == 0) L.red[tid >> 6] = pa;
    } else if (tid < HD + CS) {
        // beta enters P = T diag(beta) and L = diag(beta) A
        const int r = tid - HD;
        float db = 0.f;
        for (int s = 0; s < CS; ++s) db += L.dP[s][r] * F.T[s][r] + L.dL[r][s] * F.A[r][s];
        if (r < len) {
            const float b = F.beta[r];
            dbeta[(size_t)(t0 + r) * H + h] = tobf16(db * b * (1.f - b));
        }
    }
    __syncthreads();
    if (tid == 0) part_alog[sh] = L.red[0] + L.red[1];
}

// ---------------------------------------------------------------------------
// reduce: per head, the parameter gradients summed over chunk slots in slot
// order (128 threads: one channel each; dA_log by a fixed tree).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(HD) void bwd_reduce_kernel(
    const float *__restrict__ part_alog, const float *__restrict__ part_dtb, int64_t slots,
    int H, float *__restrict__ dA_log, float *__restrict__ ddt_bias)
{
    __shared__ float red[HD];
    const int h = blockIdx.x, c = threadIdx.x;
    float s = 0.f, a = 0.f;
    for (int64_t sl = 0; sl < slots; ++sl) s += part_dtb[((size_t)sl * H + h) * HD + c];
    for (int64_t sl = c; sl < slots; sl += HD) a += part_alog[(size_t)sl * H + h];
    if (ddt_bias) ddt_bias[(size_t)h * HD + c] = s;
    red[c] = a;
    __syncthreads();
    for (int o = HD / 2; o >= 1; o >>= 1) {
        if (c < o) red[c] += red[c + o];
        __syncthreads();
    }
    if (c == 0) dA_log[h] = red[0];
}

}  // namespace

size_t bwd_workspace_bytes(int64_t num_slots, int H) {
    const size_t sh = (size_t)num_slots * H;
    return sh * ((size_t)BR_FLOATS + 2 * (size_t)HD * HD + 1 + HD) * sizeof(float);
}

hipError_t launch_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                      const uint16_t *beta, float scale, const float *A_log,
                      const float *dt_bias, float lower_bound, const int32_t *cu, int N, int T,
                      int H, int64_t num_slots, const void *init, int init_fp32,
                      const uint16_t *dout, const float *dfin, uint16_t *dq, uint16_t *dk,
                      uint16_t *dv, uint16_t *dg, uint16_t *dbeta, float *dA_log,
                      float *ddt_bias, float *dinit, void *ws, hipStream_t stream)
{
    const size_t sh = (size_t)num_slots * H;
    float *brec = (float *)ws;
    float *st0 = brec + sh * BR_FLOATS;
    float *dst1 = st0 + sh * HD * HD;
    float *pdtb = dst1 + sh * HD * HD;
    float *palog = pdtb + sh * HD;
    const dim3 chunks((unsigned)sh), scans((unsigned)((size_t)N * H * NPART));
    hipLaunchKernelGGL(bwd_prep_kernel, chunks, dim3(BT), 0, stream,
                       q, k, g, beta, A_log, dt_bias, lower_bound, cu, N, T, H, brec);
    hipLaunchKernelGGL(bwd_states_kernel, scans, dim3(BT), 0, stream,
                       v, brec, cu, N, T, H, init, init_fp32, st0);
    hipLaunchKernelGGL(bwd_dstates_kernel, scans, dim3(BT), 0, stream,
                       dout, brec, cu, N, T, H, scale, dfin, dst1, dv, dinit);
    hipLaunchKernelGGL(bwd_chunk_kernel, chunks, dim3(BT), 0, stream,
                       q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, dout, cu, N, T, H,
                       st0, dst1, dq, dk, dg, dbeta, palog, pdtb);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)H), dim3(HD), 0, stream,
                       palog, pdtb, num_slots, H, dA_log, ddt_bias);
    return hipGetLastError();
}

}  // namespace kda
