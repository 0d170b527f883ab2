// Intra-chunk stage: token-parallel over (chunk, head).
//
// One wave handles one (16-token chunk, head); a 256-thread workgroup holds
// four consecutive heads of the same chunk so every token row it touches is
// one contiguous 1 KB run of q / k / g.  Per chunk it
//   1. evaluates the gate in base 2 (the exponent rebasing idea of "Moonshot
//      AI Open-Sources FlashKDA", section "What makes the kernel fast"):
//        log2 alpha = max(-A * log2(1 + 2^{(g + dt_bias) log2 e}), lb log2 e)
//      and beta = sigmoid(logit);
//   2. takes the in-chunk inclusive cumulative sum G of log2 alpha;
//   3. forms Kt = k 2^G, Qt = q 2^G, Kb = k 2^-G (bf16, via LDS);
//   4. A_kk = Kt Kb^T, its transpose and Aqk^T on bf16 MFMA;
//   5. T = (I + diag(beta) strict_lower(A_kk))^{-1} by the product form of
//      the Neumann series of a nilpotent matrix,
//        (I - N)^{-1} = (I + N)(I + N^2)(I + N^4)(I + N^8),  N^16 = 0,
//      on fp32 16x16x4 MFMAs (the small-inverse step of the same section);
//   6. writes the hand-off record the scan consumes.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int WAVES = 4;
constexpr int LROW = 136;   // bf16 per LDS row: 128 + 8 padding (conflict-free row-strided reads)

// Z = X Y for 16x16 fp32 matrices held in MFMA accumulator layout: xt is the
// accumulator layout of X^T (equal to the A-operand layout of X) and y that
// of Y (equal to its B-operand layout).  MFMA j takes k = 4(l/16) + j.
__device__ __forceinline__ f32x4_t mm16(f32x4_t xt, f32x4_t y) {
    f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    z = mfma_k4(xt[0], y[0], z);
    z = mfma_k4(xt[1], y[1], z);
    z = mfma_k4(xt[2], y[2], z);
    z = mfma_k4(xt[3], y[3], z);
    return z;
}

__device__ __forceinline__ float elem(const u32x4_t &v, int i) {
    uint32_t w = v[i >> 1];
    return (i & 1) ? bf16hi(w) : bf16lo(w);
}

__global__ __launch_bounds__(256) void intra_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ g, const uint16_t *__restrict__ beta,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float lb2,
    const int32_t *__restrict__ cu, int N, int T, int H, uint8_t *__restrict__ ws)
{
    __shared__ __attribute__((aligned(16))) uint16_t sK[WAVES][CS][LROW];
    __shared__ __attribute__((aligned(16))) uint16_t sQ[WAVES][CS][LROW];
    __shared__ __attribute__((aligned(16))) uint16_t sB[WAVES][CS][LROW];
    __shared__ float sBeta[WAVES][CS];

    const int w = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int grp = l >> 4;        // token group: rows 4grp .. 4grp+3 while loading
    const int cg = l & 15;         // channel group: channels 8cg .. 8cg+7 while loading
    const int64_t slot = blockIdx.x;
    const int h = blockIdx.y * WAVES + w;
    const bool hv = h < H;         // wave-uniform
    const int hh = hv ? h : 0;

    // Which sequence owns this slot: largest n with slot0(n) <= slot.
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (seq_slot0(cu, mid, T) <= slot) lo = mid; else hi = mid - 1;
    }
    const int n = lo;
    int64_t start, end;
    seq_range(cu, n, T, start, end);
    const int64_t t0 = start + (slot - seq_slot0(cu, n, T)) * CS;
    if (t0 >= end) return;                         // gap slot, block-uniform
    const int len = (int)min((int64_t)CS, end - t0);
    uint8_t *rec = ws + ((size_t)slot * H + hh) * REC_BYTES;

    // ---- gate parameters -------------------------------------------------
    const float A = expf(A_log[hh]);
    float dtb2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        dtb2[i] = dt_bias ? dt_bias[(size_t)hh * HD + 8 * cg + i] * LOG2E : 0.f;

    if (l < CS) {
        float b = 0.f;
        if (hv && l < len) {
            float x = bf16f(beta[(size_t)(t0 + l) * H + hh]);
            b = __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * LOG2E));
        }
        sBeta[w][l] = b;
    }

    // ---- load rows 4grp+p, channels 8cg..8cg+7 ----------------------------
    u32x4_t rg[4], rq[4], rk[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = 4 * grp + p;
        const u32x4_t z = {0u, 0u, 0u, 0u};
        rg[p] = z; rq[p] = z; rk[p] = z;
        if (hv && r < len) {
            const size_t off = ((size_t)(t0 + r) * H + hh) * HD + 8 * cg;
            rg[p] = *(const u32x4_t *)(g + off);
            rq[p] = *(const u32x4_t *)(q + off);
            rk[p] = *(const u32x4_t *)(k + off);
        }
    }

    // ---- gate and in-lane cumulative sum ---------------------------------
    float G[4][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float x2 = elem(rg[p], i) * LOG2E + dtb2[i];
            const float u = x2 > 64.f ? x2 : fast_log2(1.f + fast_exp2(x2));
            const float la = fmaxf(-A * u, lb2);
            acc += (4 * grp + p < len) ? la : 0.f;
            G[p][i] = acc;
        }
    }
    // exclusive prefix over the four token groups (lanes 16 apart)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float tot = G[3][i];
        float s1 = __shfl_up(tot, 16);
        float inc = tot + (grp >= 1 ? s1 : 0.f);
        float s2 = __shfl_up(inc, 32);
        inc = inc + (grp >= 2 ? s2 : 0.f);
        float ex = __shfl_up(inc, 16);
        ex = grp >= 1 ? ex : 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) G[p][i] += ex;
    }

    // ---- decayed operands ------------------------------------------------
    u32x4_t kt4[4], qt4[4], kb4[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float kt[8], qt[8], kb[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float eg = fast_exp2(G[p][i]);
            const float egi = fast_exp2(-G[p][i]);
            const float kv = elem(rk[p], i), qv = elem(rq[p], i);
            kt[i] = kv * eg;
            qt[i] = qv * eg;
            kb[i] = kv * egi;
        }
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            kt4[p][wd] = pack2(kt[2 * wd], kt[2 * wd + 1]);
            qt4[p][wd] = pack2(qt[2 * wd], qt[2 * wd + 1]);
            kb4[p][wd] = pack2(kb[2 * wd], kb[2 * wd + 1]);
        }
        const int r = 4 * grp + p;
        *(u32x4_t *)&sK[w][r][8 * cg] = kt4[p];
        *(u32x4_t *)&sQ[w][r][8 * cg] = qt4[p];
        *(u32x4_t *)&sB[w][r][8 * cg] = kb4[p];
    }

    if (hv) {
        // decay over the whole chunk (rows past len contribute nothing)
        if (grp == 3) {
            f32x4_t g0, g1;
#pragma unroll
            for (int i = 0; i < 4; ++i) { g0[i] = fast_exp2(G[3][i]); g1[i] = fast_exp2(G[3][4 + i]); }
            float *gp = (float *)(rec + REC_GAM) + 8 * cg;
            *(f32x4_t *)gp = g0;
            *(f32x4_t *)(gp + 4) = g1;
        }
        // Kb^T tiles straight from registers: channel 8cg+i lands in state
        // tile t = 2(cg/4) + i/4, row rho = 4(cg%4) + i%4, consumer lane
        // 16grp + rho; channels i and i+4 share one 16-byte slot.
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            auto half = [&](int i, int p) -> uint32_t {
                uint32_t wd = kb4[p][i >> 1];
                return (i & 1) ? (wd >> 16) : (wd & 0xffffu);
            };
            u32x4_t o;
            o[0] = half(jj, 0) | (half(jj, 1) << 16);
            o[1] = half(jj, 2) | (half(jj, 3) << 16);
            o[2] = half(jj + 4, 0) | (half(jj + 4, 1) << 16);
            o[3] = half(jj + 4, 2) | (half(jj + 4, 3) << 16);
            const int m = 16 * grp + 4 * (cg & 3) + jj;
            *(u32x4_t *)(rec + REC_KB + ((cg >> 2) * 64 + m) * 16) = o;
        }
    }

    __syncthreads();

    // ---- in-chunk products on bf16 MFMA ----------------------------------
    // MFMA view: lane l is row cg (token), k-slots 8grp..8grp+7.
    f32x4_t Akk = {0.f, 0.f, 0.f, 0.f}, AkkT = Akk, AqkT = Akk;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const u32x4_t aK = *(const u32x4_t *)&sK[w][cg][32 * kb + 8 * grp];
        const u32x4_t aQ = *(const u32x4_t *)&sQ[w][cg][32 * kb + 8 * grp];
        const u32x4_t aB = *(const u32x4_t *)&sB[w][cg][32 * kb + 8 * grp];
        if (hv) {
            *(u32x4_t *)(rec + REC_KT + (kb * 64 + l) * 16) = aK;
            *(u32x4_t *)(rec + REC_QT + (kb * 64 + l) * 16) = aQ;
        }
        Akk = mfma_k32(aK, aB, Akk);     // Akk[4grp+j][cg]    = Kt_r . Kb_i
        AkkT = mfma_k32(aB, aK, AkkT);   // AkkT[4grp+j][cg]   = Akk[cg][4grp+j]
        AqkT = mfma_k32(aB, aQ, AqkT);   // AqkT[4grp+j][cg]   = Aqk[cg][4grp+j]
    }

    // ---- T = (I + L)^{-1}, L = diag(beta) strict_lower(Akk) ---------------
    float br[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) br[j] = sBeta[w][4 * grp + j];
    const float bc = sBeta[w][cg];
    f32x4_t N1, N1t, I;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * grp + j;            // accumulator row of this lane
        N1[j] = (cg < r) ? -br[j] * Akk[j] : 0.f;
        N1t[j] = (r < cg) ? -bc * AkkT[j] : 0.f;
        I[j] = (r == cg) ? 1.f : 0.f;
    }
    const f32x4_t P1 = I + N1, P1t = I + N1t;
    const f32x4_t N2 = mm16(N1t, N1), N2t = mm16(N1, N1t);
    const f32x4_t P2 = I + N2;
    const f32x4_t Q12 = mm16(P1t, P2), Q12t = mm16(P2, P1t);
    (void)Q12;
    const f32x4_t N4 = mm16(N2t, N2), N4t = mm16(N2, N2t);
    const f32x4_t P4 = I + N4;
    const f32x4_t Q3t = mm16(P4, Q12t);                 // ((I+N)(I+N^2)(I+N^4))^T
    const f32x4_t N8 = mm16(N4t, N4);
    const f32x4_t P8 = I + N8;
    const f32x4_t Tt = mm16(P8, Q3t);                   // T^T in accumulator layout

    if (hv) {
        // A-operand layouts: lane l holds row cg, k = 4grp + j.
        u32x4_t ta;
        ta[0] = pack2(Tt[0] * br[0], Tt[1] * br[1]);     // T diag(beta)
        ta[1] = pack2(Tt[2] * br[2], Tt[3] * br[3]);
        float aq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) aq[j] = (4 * grp + j <= cg) ? AqkT[j] : 0.f;
        ta[2] = pack2(aq[0], aq[1]);
        ta[3] = pack2(aq[2], aq[3]);
        *(u32x4_t *)(rec + REC_TA + l * 16) = ta;
    }
}

}  // namespace

hipError_t launch_intra(const uint16_t *q, const uint16_t *k, const uint16_t *g,
                        const uint16_t *beta, const float *A_log, const float *dt_bias,
                        float lower_bound, const int32_t *cu, int N, int T, int H,
                        int64_t num_slots, uint8_t *ws, hipStream_t stream)
{
    if (num_slots <= 0) return hipSuccess;
    dim3 grid((unsigned)num_slots, (unsigned)((H + WAVES - 1) / WAVES));
    hipLaunchKernelGGL(intra_kernel, grid, dim3(64 * WAVES), 0, stream,
                       q, k, g, beta, A_log, dt_bias, lower_bound * LOG2E, cu, N, T, H, ws);
    return hipGetLastError();
}

}  // namespace kda
