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
// Five launches:
//   prep    (chunk slot, head)  the chunk factors in fp32: Kt and Wm (with the
//           chunk decay) for the states scan, and the reverse scan's bf16
//           record (Wm, scale Qt, -Kt, scale M^T in MFMA operand layouts)
//   states  (sequence, head, four 16-column parts)  forward scan storing
//           every chunk's start state S0 and X (fp32 16x16x4 MFMA)
//   rscan   (sequence, head, column part)  reverse scan of dS on the forward
//           scan's structure (kda_scan.hip: bf16 MFMA operands, fp32
//           accumulators), storing every chunk's dS1 (bf16) and dX,
//           writing dv and the initial-state gradient
//   chunk   (chunk slot, head)  the products with S0 / dS1 (fp32 MFMA) and
//           the in-chunk backward: dq, dk, dg, dbeta, per-chunk dA_log /
//           ddt_bias sums
//   reduce  (head)  sums the per-chunk parameter gradients in slot order
// Every sum runs in a fixed order, so results are bitwise reproducible.
#include <math.h>

#include "kda_device.h"
#include "kda_intra_dev.h"                            // mm16: 16 x 16 fp32 products on MFMA
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int BT = 256;               // threads per workgroup
constexpr int RS = HD + 4;            // padded LDS row stride (floats)
constexpr int SP = CS + 1;            // padded stride of 16 x 16 tiles
constexpr int CWB = 16;               // state columns of one stored part
constexpr int NPART = HD / CWB;

// The transcendentals on the hardware base-2 units (v_exp_f32, v_log_f32,
// v_rcp_f32).  softplus keeps the form max(x, 0) + log(1 + e^-|x|), finite
// for every finite x, so that -exp(A_log) softplus(x) is -0, not NaN, when
// A_log = -inf.
constexpr float LN2 = 0.6931471805599453f;
__device__ __forceinline__ float softplus_f(float x) {
    return fmaxf(x, 0.f) + LN2 * fast_log2(1.f + fast_exp2(-fabsf(x) * LOG2E));
}
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * LOG2E));
}
__device__ __forceinline__ float exp_f(float x) { return fast_exp2(x * LOG2E); }

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
struct FactorsBase {
    float kt[CS][RS], qt[CS][RS], kb[CS][RS], e[CS][RS];
    float A[CS][SP], aqk[CS][SP], T[CS][SP], P[CS][SP], M[CS][SP];
    float beta[CS], gam[HD], dtb[HD];
};
struct Factors : FactorsBase {
    float wm[CS][RS];                 // Wm = P^T Kb Gam (the prep kernel's record)
};

// WANT_W: also form Wm in L.wm (L a Factors; the prep kernel stores it).  The
// chunk kernel does not use Wm and passes a FactorsBase.
// KEEP_GATE: also return, per row, the gate before its clamp,
// y = -exp(A_log) softplus(g + dt_bias), and sigmoid(g + dt_bias) in ysv /
// sgv (the calling thread's channel, threads below HD), for the gate chain
// of the chunk kernel.
template <bool WANT_W, bool KEEP_GATE = false, class FL>
__device__ __forceinline__ void chunk_factors(FL &L, const uint16_t *__restrict__ q,
                              const uint16_t *__restrict__ k, const uint16_t *__restrict__ g,
                              const uint16_t *__restrict__ bl, float Aexp,
                              const float *__restrict__ dt_bias, float lb, int64_t t0, int len,
                              int H, int h, int kd, float *ysv = nullptr, float *sgv = nullptr) {
    const int tid = threadIdx.x;
    if (tid < HD) {
        // one channel per thread: gate, in-chunk cumulative log-decay G
        // (natural log) and the scaled rows
        const int c = tid;
        // head dimension kd = 64 runs on the 128-wide tiles: channels from kd
        // on have zero k and q (and zero gate inputs), so every factor row
        // and column they touch is zero
        const bool ch = c < kd;
        const int cc = ch ? c : 0;                   // an address that is always in range
        const float dtb = (dt_bias && ch) ? dt_bias[(size_t)h * kd + c] : 0.f;
        L.dtb[c] = dtb;
        // every row's loads first and unconditionally, so that their
        // latencies overlap (rows past len read row len-1; both are masked
        // after the loads)
        uint16_t gw[CS], kw[CS], qw[CS];
#pragma unroll
        for (int r = 0; r < CS; ++r) {
            const size_t off = ((size_t)(t0 + (r < len ? r : len - 1)) * H + h) * kd + cc;
            gw[r] = g[off];
            kw[r] = k[off];
            qw[r] = q[off];
        }
        float gr[CS], kr[CS], qr[CS];
#pragma unroll
        for (int r = 0; r < CS; ++r) {
            gr[r] = ch ? bf16f(gw[r]) : 0.f;
            kr[r] = ch ? bf16f(kw[r]) : 0.f;
            qr[r] = ch ? bf16f(qw[r]) : 0.f;
        }
        float G = 0.f;
#pragma unroll
        for (int r = 0; r < CS; ++r) {
            float kv = 0.f, qv = 0.f;
            if (r < len) {
                const float y = -Aexp * softplus_f(gr[r] + dtb);
                if (KEEP_GATE) {
                    ysv[r] = y;
                    sgv[r] = sigmoid_f(gr[r] + dtb);
                }
                G += fmaxf(y, lb);
                kv = kr[r];
                qv = qr[r];
            }
            const float e = exp_f(G);
            L.e[r][c] = e;
            L.kt[r][c] = kv * e;
            L.qt[r][c] = qv * e;
            L.kb[r][c] = kv * exp_f(-G);
        }
        L.gam[c] = L.e[CS - 1][c];
    } else if (tid < HD + CS) {
        const int r = tid - HD;
        L.beta[r] = r < len ? sigmoid_f(bf16f(bl[(size_t)(t0 + r) * H + h])) : 0.f;
    }
    __syncthreads();
    {
        // A = strict_lower(Kt Kb^T) on wave 0, Aqk = lower_incl(Qt Kb^T) on
        // wave 1: fp32 16x16x4 MFMAs over the 128 channels (lane l supplies
        // row l%16, channel 4ks + l/16 of each operand and holds rows
        // 4(l/16) .. +3, column l%16 of the product)
        const int wave = tid >> 6, l = tid & 63;
        if (wave < 2) {
            const float(&lhs)[CS][RS] = wave == 0 ? L.kt : L.qt;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
            for (int ks = 0; ks < HD / 4; ++ks)
                acc = mfma_k4(lhs[l & 15][4 * ks + (l >> 4)], L.kb[l & 15][4 * ks + (l >> 4)], acc);
            const int i = l & 15;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * (l >> 4) + j;
                if (wave == 0) L.A[r][i] = i < r ? acc[j] : 0.f;
                else L.aqk[r][i] = i <= r ? acc[j] : 0.f;
            }
        }
    }
    __syncthreads();
    if (tid < 64) {
        // T = (I + diag(beta) A)^-1 = (I - N)^-1 with N = -diag(beta) A
        // strictly lower, hence nilpotent: (I + N)(I + N^2)(I + N^4)(I + N^8),
        // on fp32 16x16x4 MFMAs in one wave.  Lane l holds rows 4(l/16) + j,
        // column l%16 of each matrix and of its transpose (the A-operand
        // layout of the matrix itself).
        const int l = tid, grp = l >> 4, cg = l & 15;
        f32x4_t N1, N1t, I;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * grp + j;
            N1[j] = -L.beta[r] * L.A[r][cg];          // A is zero on and above the diagonal
            N1t[j] = -L.beta[cg] * L.A[cg][r];
            I[j] = r == cg ? 1.f : 0.f;
        }
        const f32x4_t P1t = I + N1t;
        const f32x4_t N2 = mm16(N1t, N1), N2t = mm16(N1, N1t);
        const f32x4_t Q12t = mm16(I + N2, P1t);       // ((I+N)(I+N^2))^T
        const f32x4_t N4 = mm16(N2t, N2), N4t = mm16(N2, N2t);
        const f32x4_t Q3t = mm16(I + N4, Q12t);       // ((I+N)(I+N^2)(I+N^4))^T
        const f32x4_t N8 = mm16(N4t, N4);
        const f32x4_t Tm = mm16(Q3t, I + N8);
#pragma unroll
        for (int j = 0; j < 4; ++j) L.T[4 * grp + j][cg] = Tm[j];
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
        if constexpr (WANT_W) {
            // Wm = P^T Kb Gam on fp32 16x16x4 MFMAs, wave w taking channel
            // tiles 2w and 2w+1 (lane l: A = P^T row l%16, token 4ks + l/16;
            // B = Kb token 4ks + l/16, channel l%16; result rows 4(l/16) + j)
            const int wave = tid >> 6, l = tid & 63;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int c = 16 * (2 * wave + tt) + (l & 15);
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    acc = mfma_k4(L.P[4 * ks + (l >> 4)][l & 15], L.kb[4 * ks + (l >> 4)][c], acc);
                const float gc = L.gam[c];
#pragma unroll
                for (int j = 0; j < 4; ++j) L.wm[4 * (l >> 4) + j][c] = acc[j] * gc;
            }
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// prep: the chunk factors in fp32, into the two scans' bf16 records (in the
// forward record's MFMA operand layouts, RecLayout<HD>):
//   states record (StatesRec): Kt and Wm = P^T Kb Gam as (hi, lo) bf16
//     pairs in the Kt and W^T layouts, and the chunk decay, the operands of
//     X = V - Kt S0 and S1 = Gam S0 + Wm^T X;
//   reverse record: Wm as the A operand of Wm dS (the Kt slot), scale Qt
//     and -Kt transposed as the A operands of the state-gradient update (the
//     Qt and W^T slots, both in the W^T layout), scale M^T (the M slot) and
//     the chunk decay.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(BT) void bwd_prep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ g, const uint16_t *__restrict__ beta,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float lb, float scale,
    const int32_t *__restrict__ cu, int N, int T, int H, int kd, uint8_t *__restrict__ srec,
    uint8_t *__restrict__ rrec)
{
    __shared__ __attribute__((aligned(16))) Factors L;
    const int64_t slot = blockIdx.x / (unsigned)H;
    const int h = (int)(blockIdx.x % (unsigned)H);
    int64_t t0;
    const int len = slot_chunk(cu, N, T, slot, t0);
    if (len == 0) return;                                   // gap slot
    chunk_factors<true>(L, q, k, g, beta, expf(A_log[h]), dt_bias, lb, t0, len, H, h, kd);
    const int tid = threadIdx.x;

    typedef RecLayout<HD> R;
    typedef StatesRec SR;
    uint8_t *sr = srec + ((size_t)slot * H + h) * SR::BYTES;
    uint8_t *rr = rrec + ((size_t)slot * H + h) * R::BYTES;
    uint16_t *s_kt = (uint16_t *)(sr + SR::KTH), *s_ktl = (uint16_t *)(sr + SR::KTL);
    uint16_t *s_wt = (uint16_t *)(sr + SR::WTH), *s_wtl = (uint16_t *)(sr + SR::WTL);
    uint16_t *r_kt = (uint16_t *)(rr + R::KTO), *r_qt = (uint16_t *)(rr + R::QT);
    uint16_t *r_wt = (uint16_t *)(rr + R::WT), *r_m = (uint16_t *)(rr + R::M);
    // Kt slot: element (kb, lane l, i) = X[l%16][32 kb + 8 (l/16) + i]
    // W^T-layout slots: element (tp, lane l, 4 hf + j) = X[4 (l/16) + j][chan(2 tp + hf, l%16)]
    for (int e = tid; e < 4 * 64 * 8; e += BT) {
        const int kb = e >> 9, l = (e >> 3) & 63, i = e & 7;
        const int ck = 32 * kb + 8 * (l >> 4) + i;
        const float ktv = L.kt[l & 15][ck];
        s_kt[e] = tobf16(ktv);
        s_ktl[e] = tobf16(ktv - bf16f(s_kt[e]));
        r_kt[e] = tobf16(L.wm[l & 15][ck]);
        const int tok = 4 * (l >> 4) + (i & 3), ch = state_chan(2 * kb + (i >> 2), l & 15);
        const float wmv = L.wm[tok][ch];
        s_wt[e] = tobf16(wmv);
        s_wtl[e] = tobf16(wmv - bf16f(s_wt[e]));
        r_qt[e] = tobf16(scale * L.qt[tok][ch]);
        r_wt[e] = tobf16(-L.kt[tok][ch]);
    }
    // M slot: element (lane l, j) = scale M[4 (l/16) + j][l%16]
    r_m[tid] = tobf16(scale * L.M[4 * ((tid >> 2) >> 4) + (tid & 3)][(tid >> 2) & 15]);
    if (tid < HD) {
        ((float *)(sr + SR::GAM))[tid] = L.gam[tid];
        ((float *)(rr + R::GAM))[tid] = L.gam[tid];
    }
}


// ---------------------------------------------------------------------------
// chunk: per (chunk slot, head), everything that needs S0 and dS1 of the
// chunk, then the in-chunk backward down to the inputs.
// ---------------------------------------------------------------------------
// Buffers whose lifetimes do not overlap share storage, which keeps the
// workgroup at 73 KB of LDS (two workgroups per compute unit):
//   dol  scale * dO: the state products and dM; then dG of every (row, channel)
//   xl   X: the state products and dM
//   u    dX for the state products; then the 16 x 16 gradient tiles
//   dwm  dWm: written by the state products, read by the later phases
struct ChunkTiles {
    float dM[CS][SP], dAqk[CS][SP], dP[CS][SP], Y[CS][SP], dL[CS][SP], dA[CS][SP];
};
struct ChunkLds {
    FactorsBase f;
    float dol[CS][RS], xl[CS][RS];
    union {
        float dxl[CS][RS];
        ChunkTiles t;
    } u;
    float dwm[CS][RS];
    float dgam[HD], dgam2[HD], red[BT / 64];
};
static_assert(2 * sizeof(ChunkLds) <= 160 * 1024, "two chunk workgroups per compute unit");

// Row r (a channel) of the 16-channel block cb of a stored state (S0 or
// dS1, which the backward's scans store in bf16 as rows of each 16-column
// part, [part][128 rows][16 columns]) as the B operand of eight 16x16x4
// k-step groups: lane (r, j) loads, from each part p, the four columns
// 16 p + 4 j .. + 3 (8 bytes, widened).  Parts from np on (columns past the
// head dimension) are not stored and read as zeros; their loads are issued
// anyway (at part 0) so that no branch forces a wait on the loads in flight.
__device__ __forceinline__ void fetch_state_rows(float4 (&d)[NPART], const uint16_t *__restrict__ base,
                                                 int cb, int l, int np) {
    const int r = l & 15, j = l >> 4;
#pragma unroll
    for (int p = 0; p < NPART; ++p) {
        const int pp = p < np ? p : 0;
        const u32x2_t w = *(const u32x2_t *)&base[((size_t)pp * HD + 16 * cb + r) * 16 + 4 * j];
        const bool in = p < np;
        d[p] = make_float4(in ? bf16lo(w[0]) : 0.f, in ? bf16hi(w[0]) : 0.f,
                           in ? bf16lo(w[1]) : 0.f, in ? bf16hi(w[1]) : 0.f);
    }
}

__global__ __launch_bounds__(BT, 2) void bwd_chunk_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ g, const uint16_t *__restrict__ beta,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float lb, float scale,
    const uint16_t *__restrict__ dout, const int32_t *__restrict__ cu, int N, int T, int H, int kd,
    const uint16_t *__restrict__ st0, const uint16_t *__restrict__ dst1,
    const float *__restrict__ xws, const float *__restrict__ dxws,
    uint16_t *__restrict__ dq, uint16_t *__restrict__ dk, uint16_t *__restrict__ dg,
    uint16_t *__restrict__ dbeta, float *__restrict__ part_alog, float *__restrict__ part_dtb)
{
    __shared__ __attribute__((aligned(16))) ChunkLds L;
    FactorsBase &F = L.f;
    ChunkTiles &Lt = L.u.t;
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
    const uint16_t *S0 = st0 + sh * HD * HD;
    const uint16_t *DS = dst1 + sh * HD * HD;
    const int np = kd / CWB;                                // stored parts of S0 and dS1
    // Wave w takes the 16-channel blocks 2w and 2w + 1 of S0 and dS1; the
    // first block's rows are in flight during the factors.
    const int wave = tid >> 6, l = tid & 63;
    float4 sb[NPART], db[NPART];
    fetch_state_rows(sb, S0, 2 * wave, l, np);
    fetch_state_rows(db, DS, 2 * wave, l, np);
    const float Aexp = expf(A_log[h]);
    float ysv[CS], sgv[CS];                                 // this thread's gate per row (threads < HD)
    chunk_factors<false, true>(F, q, k, g, beta, Aexp, dt_bias, lb, t0, len, H, h, kd, ysv, sgv);

    {
        // all eight loads of this thread first (rows past len read row
        // len-1 and are masked)
        uint16_t dov[CS * HD / BT];
#pragma unroll
        for (int m = 0; m < CS * HD / BT; ++m) {
            const int idx = tid + m * BT, r = idx / HD, c = idx % HD;
            dov[m] = dout[((size_t)(t0 + (r < len ? r : len - 1)) * H + h) * kd + (c < kd ? c : 0)];
        }
#pragma unroll
        for (int m = 0; m < CS * HD / BT; ++m) {
            const int idx = tid + m * BT, r = idx / HD, c = idx % HD;
            L.dol[r][c] = (r < len && c < kd) ? scale * bf16f(dov[m]) : 0.f;
        }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        // X and dX; the columns past the head dimension are not stored by
        // the reverse scan and are zeros here
        const int e = 4 * (tid + m * BT);
        const bool cv = e % HD < kd;
        const float4 xv = *(const float4 *)&xws[sh * CS * HD + e];
        const float4 dxv = *(const float4 *)&dxws[sh * CS * HD + e];
        *(float4 *)&L.xl[e / HD][e % HD] =
            make_float4(cv ? xv.x : 0.f, cv ? xv.y : 0.f, cv ? xv.z : 0.f, cv ? xv.w : 0.f);
        *(float4 *)&L.u.dxl[e / HD][e % HD] =
            make_float4(cv ? dxv.x : 0.f, cv ? dxv.y : 0.f, cv ? dxv.z : 0.f, cv ? dxv.w : 0.f);
    }
    __syncthreads();

    // Products with the states on fp32 16x16x4 MFMAs, contracting over the
    // 128 value columns; wave w forms them for channel blocks cb = 2w + tt:
    //   dQt = scale dO S0^T,  dKt = -dX S0^T,  dWm = X dS1^T,
    //   dGam = diag(dS1 S0^T) (vector ALUs, summed over the four lane groups).
    // k-step 4p + i takes column 16p + 4(l/16) + i from lane l (the order of the
    // state rows as loaded); the A operands follow the same order.  Lane l
    // holds rows 4(l/16) .. +3, channel 16cb + l%16 of each product, the
    // layout of the per-(row, channel) phase below, so dQt and dKt stay in
    // registers.
    f32x4_t dQs[2], dKs[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int cb = 2 * wave + tt;
        float4 sn[NPART], dn[NPART];
        if (tt == 0) {                                      // the next block in flight
            fetch_state_rows(sn, S0, cb + 1, l, np);
            fetch_state_rows(dn, DS, cb + 1, l, np);
        }
        f32x4_t aq = {0.f, 0.f, 0.f, 0.f}, ak = aq, aw = aq;
        float pg = 0.f;
#pragma unroll
        for (int p = 0; p < NPART; ++p) {
            const int c0 = 16 * p + 4 * (l >> 4);
            const float4 ad = *(const float4 *)&L.dol[l & 15][c0];
            const float4 ax = *(const float4 *)&L.u.dxl[l & 15][c0];
            const float4 aX = *(const float4 *)&L.xl[l & 15][c0];
            aq = mfma_k4(ad.x, sb[p].x, aq);
            aq = mfma_k4(ad.y, sb[p].y, aq);
            aq = mfma_k4(ad.z, sb[p].z, aq);
            aq = mfma_k4(ad.w, sb[p].w, aq);
            ak = mfma_k4(-ax.x, sb[p].x, ak);
            ak = mfma_k4(-ax.y, sb[p].y, ak);
            ak = mfma_k4(-ax.z, sb[p].z, ak);
            ak = mfma_k4(-ax.w, sb[p].w, ak);
            aw = mfma_k4(aX.x, db[p].x, aw);
            aw = mfma_k4(aX.y, db[p].y, aw);
            aw = mfma_k4(aX.z, db[p].z, aw);
            aw = mfma_k4(aX.w, db[p].w, aw);
            pg += db[p].x * sb[p].x + db[p].y * sb[p].y + db[p].z * sb[p].z + db[p].w * sb[p].w;
        }
        dQs[tt] = aq;
        dKs[tt] = ak;
#pragma unroll
        for (int i = 0; i < 4; ++i) L.dwm[4 * (l >> 4) + i][16 * cb + (l & 15)] = aw[i];
        pg += __shfl_xor(pg, 16, 64);
        pg += __shfl_xor(pg, 32, 64);
        if ((l >> 4) == 0) L.dgam[16 * cb + (l & 15)] = pg;
        if (tt == 0) {
#pragma unroll
            for (int p = 0; p < NPART; ++p) {
                sb[p] = sn[p];
                db[p] = dn[p];
            }
        }
    }
    // dWm complete and dX no longer read (its storage holds the 16 x 16 tiles next)
    __syncthreads();
    const int r_ = tid >> 4, lo = tid & 15;
    {
        // The two contractions over 128 channels on fp32 16x16x4 MFMAs:
        // wave 0 dM = scale dO X^T, wave 1 the Wm path of dP, Kb Gam dWm^T
        // (held in Y, which is free until the phase after next).  Lane l
        // supplies row l%16, channel 4ks + l/16 of both operands and holds
        // rows 4(l/16) .. +3, column l%16.
        const int ar = l & 15, ak = l >> 4;
        if (wave < 2) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            if (wave == 0) {
#pragma unroll 8
                for (int ks = 0; ks < HD / 4; ++ks)
                    acc = mfma_k4(L.dol[ar][4 * ks + ak], L.xl[ar][4 * ks + ak], acc);
            } else {
#pragma unroll 8
                for (int ks = 0; ks < HD / 4; ++ks) {
                    const int c = 4 * ks + ak;
                    acc = mfma_k4(F.kb[ar][c] * F.gam[c], L.dwm[ar][c], acc);
                }
            }
            float(&dst)[CS][SP] = wave == 0 ? Lt.dM : Lt.Y;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[4 * ak + j][ar] = acc[j];
        }
    }
    __syncthreads();
    {
        // M = Aqk P:  dAqk = dM P^T (lower incl.),  dP = Aqk^T dM
        // Wm = P^T Kb Gam:  dP += Kb Gam dWm^T (from the MFMAs above)
        const int r = r_, i = lo;
        float a = 0.f, p = 0.f;
        for (int s = 0; s < CS; ++s) {
            a += Lt.dM[r][s] * F.P[i][s];
            p += F.aqk[s][r] * Lt.dM[s][i];
        }
        p += Lt.Y[r][i];
        Lt.dAqk[r][i] = i <= r ? a : 0.f;
        Lt.dP[r][i] = p;
    }
    __syncthreads();
    {
        // P = T diag(beta):  dT = dP diag(beta);  Y = dT T^T
        const int a = r_, s = lo;
        float y = 0.f;
        for (int b = 0; b < CS; ++b) y += Lt.dP[a][b] * F.beta[b] * F.T[s][b];
        Lt.Y[a][s] = y;
    }
    __syncthreads();
    {
        // T = (I + L)^-1:  dL = -T^T dT T^T (strictly lower);  L = diag(beta) A
        const int r = r_, s = lo;
        float d = 0.f;
        for (int a = 0; a < CS; ++a) d += F.T[a][r] * Lt.Y[a][s];
        d = s < r ? -d : 0.f;
        Lt.dL[r][s] = d;
        Lt.dA[r][s] = F.beta[r] * d;
    }
    __syncthreads();
    {
        // per (token row r, channel c): the gradients of Qt, Kt, Kb, then q, k, G.
        // The 16 x 16 by 16 x 128 products on fp32 16x16x4 MFMAs, wave w
        // taking channel tiles 2w and 2w+1:
        //   dQt += dAqk Kb,  dKt += dA Kb,  dKbG = P dWm,  dKb = dAqk^T Qt + dA^T Kt
        // Lane l supplies row l%16, token 4ks + l/16 of each 16 x 16 factor
        // (A operand) and token 4ks + l/16, channel l%16 of the tile (B
        // operand), and holds rows 4(l/16) .. +3, channel l%16 of each
        // product: every (row, channel) belongs to one lane, which then
        // forms its gradients elementwise.
        const int ar = l & 15, ak = l >> 4;
        float aAqk[4], aA[4], aP[4], aAqkT[4], aAT[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            aAqk[ks] = Lt.dAqk[ar][4 * ks + ak];
            aA[ks] = Lt.dA[ar][4 * ks + ak];
            aP[ks] = F.P[ar][4 * ks + ak];
            aAqkT[ks] = Lt.dAqk[4 * ks + ak][ar];
            aAT[ks] = Lt.dA[4 * ks + ak][ar];
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int c = 16 * (2 * wave + tt) + ar;   // channel of this lane
            f32x4_t dQ = {0.f, 0.f, 0.f, 0.f}, dK = dQ, dKG = dQ, dKB = dQ;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int tk = 4 * ks + ak;             // token of the B operand
                const float kbs = F.kb[tk][c], dws = L.dwm[tk][c];
                const float qts = F.qt[tk][c], kts = F.kt[tk][c];
                dQ = mfma_k4(aAqk[ks], kbs, dQ);        // dAqk zero for s > r
                dK = mfma_k4(aA[ks], kbs, dK);          // dA zero for s >= r
                dKG = mfma_k4(aP[ks], dws, dKG);
                dKB = mfma_k4(aAqkT[ks], qts, dKB);
                dKB = mfma_k4(aAT[ks], kts, dKB);
            }
            float dgc = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * ak + j;
                const float dQt = dQs[tt][j] + dQ[j], dKt = dKs[tt][j] + dK[j];
                const float dKbG = dKG[j];
                const float dKb = dKB[j] + F.gam[c] * dKbG;
                dgc += dKbG * F.kb[r][c];
                const float e = F.e[r][c];
                if (r < len && c < kd) {
                    const size_t off = ((size_t)(t0 + r) * H + h) * kd + c;
                    dq[off] = tobf16(dQt * e);
                    dk[off] = tobf16(dKt * e + dKb / e);
                }
                // dG (natural log) of this row, stored over dO
                L.dol[r][c] = dKt * F.kt[r][c] + dQt * F.qt[r][c] - dKb * F.kb[r][c];
            }
            // sum over the four row groups (lanes l, l^16, l^32, l^48)
            dgc += __shfl_xor(dgc, 16, 64);
            dgc += __shfl_xor(dgc, 32, 64);
            if (ak == 0) {
                L.dgam2[c] = dgc;
            }
        }
    }
    __syncthreads();
    if (tid < HD) {
        // reverse cumulative sum of dG is the gradient of the per-token log-decay;
        // then the gate chain
        const int c = tid;
        const float dgam = L.dgam[c] + L.dgam2[c];
        float acc = dgam * F.gam[c];
        float pdtb = 0.f, pa = 0.f;
#pragma unroll
        for (int s = CS - 1; s >= 0; --s) {
            acc += L.dol[s][c];
            if (s < len) {
                const size_t off = ((size_t)(t0 + s) * H + h) * kd + c;
                const float y = ysv[s];                 // as in chunk_factors, same thread
                const float dy = y >= lb ? acc : 0.f;
                const float dx = -dy * Aexp * sgv[s];
                if (c < kd) dg[off] = tobf16(dx);
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
        for (int s = 0; s < CS; ++s) db += Lt.dP[s][r] * F.T[s][r] + Lt.dL[r][s] * F.A[r][s];
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
    int H, int kd, float *__restrict__ dA_log, float *__restrict__ ddt_bias)
{
    __shared__ float red[HD];
    const int h = blockIdx.x, c = threadIdx.x;
    float s = 0.f, a = 0.f;
    // slot order, sixteen loads issued ahead of their adds
    int64_t sl = 0;
    for (; sl + 16 <= slots; sl += 16) {
        float pv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[i] = part_dtb[((size_t)(sl + i) * H + h) * HD + c];
#pragma unroll
        for (int i = 0; i < 16; ++i) s += pv[i];
    }
    for (; sl < slots; ++sl) s += part_dtb[((size_t)sl * H + h) * HD + c];
    for (int64_t sl = c; sl < slots; sl += HD) a += part_alog[(size_t)sl * H + h];
    if (ddt_bias && c < kd) ddt_bias[(size_t)h * kd + c] = s;
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
    return sh * ((size_t)StatesRec::BYTES + (size_t)RecLayout<HD>::BYTES +
                 2 * (size_t)HD * HD * sizeof(uint16_t) + (2 * (size_t)CS * HD + HD + 1) * sizeof(float));
}

hipError_t launch_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                      const uint16_t *beta, float scale, const float *A_log,
                      const float *dt_bias, float lower_bound, const int32_t *cu, int N, int T,
                      int H, int K, int64_t num_slots, const void *init, int init_fp32,
                      const uint16_t *dout, const float *dfin, uint16_t *dq, uint16_t *dk,
                      uint16_t *dv, uint16_t *dg, uint16_t *dbeta, float *dA_log,
                      float *ddt_bias, float *dinit, void *ws, hipStream_t stream,
                      const hipEvent_t *events)
{
    const size_t sh = (size_t)num_slots * H;
    // every region starts at a multiple of 256 bytes (each per-(slot, head)
    // size is one, the last region's aside)
    static_assert(RecLayout<HD>::BYTES % 256 == 0 && StatesRec::BYTES % 256 == 0, "256-byte regions");
    uint8_t *srec = (uint8_t *)ws;
    uint8_t *rrec = srec + sh * StatesRec::BYTES;
    uint16_t *st0 = (uint16_t *)(rrec + sh * RecLayout<HD>::BYTES);
    uint16_t *dst1 = st0 + sh * HD * HD;
    float *xws = (float *)(dst1 + sh * HD * HD);
    float *dxws = xws + sh * CS * HD;
    float *pdtb = dxws + sh * CS * HD;
    float *palog = pdtb + sh * HD;
    const dim3 chunks((unsigned)sh);
    hipError_t e = hipSuccess;
    auto mark = [&](int i) {
        if (events && events[i] && e == hipSuccess) e = hipEventRecord(events[i], stream);
    };
    mark(0);
    hipLaunchKernelGGL(bwd_prep_kernel, chunks, dim3(BT), 0, stream,
                       q, k, g, beta, A_log, dt_bias, lower_bound, scale, cu, N, T, H, K, srec, rrec);
    mark(1);
    if (e == hipSuccess)
        e = launch_bwd_fscan(v, srec, cu, N, T, H, K, init, init_fp32, st0, xws, stream);
    mark(2);
    if (e == hipSuccess)
        e = launch_bwd_rscan(dout, rrec, cu, N, T, H, K, dfin, dinit, dv, dst1, dxws, stream);
    mark(3);
    hipLaunchKernelGGL(bwd_chunk_kernel, chunks, dim3(BT), 0, stream,
                       q, k, g, beta, A_log, dt_bias, lower_bound, scale, dout, cu, N, T, H, K,
                       st0, dst1, xws, dxws, dq, dk, dg, dbeta, palog, pdtb);
    mark(4);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)H), dim3(HD), 0, stream,
                       palog, pdtb, num_slots, H, K, dA_log, ddt_bias);
    mark(5);
    const hipError_t le = hipGetLastError();
    return e != hipSuccess ? e : le;
}

}  // namespace kda
