// Intra-chunk stage: token-parallel over (chunk, head).
//
// One wave (a workgroup of its own) handles one (16-token chunk, head).  Per
// chunk it
//   1. evaluates the gate in base 2 (the exponent rebasing idea of "Moonshot
//      AI Open-Sources FlashKDA", section "What makes the kernel fast"):
//        log2 alpha = max(-A * log2(1 + 2^{(g + dt_bias) log2 e}), lb log2 e)
//      and beta = sigmoid(logit);
//   2. takes the in-chunk inclusive cumulative sum G of log2 alpha;
//   3. forms Kt = k 2^G, Qt = q 2^G, Kb = k 2^-G; Qt and Kb also as a bf16
//      (hi, lo) pair whose sum carries ~16 mantissa bits;
//   4. A_kk = Kt Kb^T on bf16 MFMA, and Aqk^T = Kb Qt^T from three bf16 MFMA
//      products (hi hi + hi lo + lo hi) so that it is fp32-accurate;
//   5. T = (I + diag(beta) strict_lower(A_kk))^{-1} by the product form of
//      the Neumann series of a nilpotent matrix,
//        (I - N)^{-1} = (I + N)(I + N^2)(I + N^4)(I + N^8),  N^16 = 0,
//      on fp32 16x16x4 MFMAs (the small-inverse step of the same section);
//   6. M = Aqk T diag(beta) and W = (T diag(beta))^T Kb diag(e^{G_last}),
//      again from (hi, lo) bf16 products, rounded to bf16 once;
//   7. writes the hand-off record the scan consumes.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

// Token-major operand tile: 16 rows (tokens) x 128 bf16 (channels) = 16
// rows of sixteen 16-byte units; unit u of row r is stored at u ^ r, so that
// both the row-wise writes of the elementwise stage and the column-block
// reads of the MFMA stage touch eight different 16-byte bank groups per
// eight lanes.
constexpr int TILE = CS * HD;                 // bf16 per tile
__device__ __forceinline__ int tile_off(int r, int u) { return r * HD + ((u ^ r) << 3); }

// Channel-major tile (128 channels x 16 tokens, 8-byte units of 4 tokens):
// channel ch sits in row slot (ch & ~3) | ((ch ^ (ch >> 5)) & 3) and its
// token unit gq in unit gq ^ ((ch >> 3) & 3).  Both the writes (lanes vary
// channel bits 3..6) and the W-operand reads (lanes vary bits 0, 1, 3, 4)
// then hit sixteen different 8-byte bank pairs per sixteen lanes.
__device__ __forceinline__ int cmaj_off(int ch, int gq) {
    const int row = (ch & ~3) | ((ch ^ (ch >> 5)) & 3);
    return row * CS + ((gq ^ ((ch >> 3) & 3)) << 2);
}

struct WaveLds {
    // Kt, Qt hi, Qt lo, Kb hi, Kb lo (token-major).  Once the Gram products
    // have read them, tiles 0 and 1 are reused for Kb hi / lo channel-major.
    uint16_t tile[5][TILE];
    float beta[CS];
    float gam[HD];                  // e^{G_last} per channel
};

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

// bf16 (hi, lo) split of two fp32 values: hi = rne(x), lo = rne(x - hi).
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pack2(a, b);
    lo = pack2(a - bf16lo(hi), b - bf16hi(hi));
}

__device__ __forceinline__ uint32_t half16(uint32_t w, int i) {
    return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

// One (chunk, head) of the intra-chunk stage by one wave.  FULL: all 16
// rows are tokens of the sequence (no masking of the cumulative decay).
template <bool FULL>
__device__ __forceinline__ void intra_chunk(
    WaveLds &L, const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ g, const uint16_t *__restrict__ beta,
    float A, const float (&dtb2)[8], float lb2, int64_t t0, int len, int H, int hh,
    uint8_t *__restrict__ rec)
{
    const int l = threadIdx.x & 63;
    const int grp = l >> 4;        // token group: rows 4grp .. 4grp+3 while loading
    const int cg = l & 15;         // channel group: channels 8cg .. 8cg+7 while loading
    const size_t row_elems = (size_t)H * HD;

    if (l < CS) {
        float b = 0.f;
        if (FULL || l < len) {
            float x = bf16f(beta[(size_t)(t0 + l) * H + hh]);
            b = __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * LOG2E));
        }
        L.beta[l] = b;
    }

    // ---- load rows 4grp+p, channels 8cg..8cg+7 (rows past len read as 0) --
    u32x4_t rg[4], rq[4], rk[4];
    {
        const size_t base = ((size_t)t0 * H + hh) * HD;
        const uint32_t bytes = (uint32_t)(((size_t)(len - 1) * row_elems + HD) * 2);
        const __amdgpu_buffer_rsrc_t sg = make_rsrc(g + base, bytes);
        const __amdgpu_buffer_rsrc_t sq = make_rsrc(q + base, bytes);
        const __amdgpu_buffer_rsrc_t sk = make_rsrc(k + base, bytes);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int off = (int)(((4 * grp + p) * row_elems + 8 * cg) * 2);
            rg[p] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sg, off, 0, 0));
            rq[p] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sq, off, 0, 0));
            rk[p] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sk, off, 0, 0));
        }
    }

    // ---- gate and cumulative sum ----------------------------------------
    // A == 0 (A_log = -inf) means no decay at all; the wave-uniform branch
    // keeps the per-element path free of 0 * inf.
    float G[4][8];
    if (A > 0.f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float x2 = elem(rg[p], i) * LOG2E + dtb2[i];
                const float u = fast_log2(1.f + fast_exp2(x2));
                const float la = fmaxf(-A * u, lb2);
                acc += (FULL || 4 * grp + p < len) ? la : 0.f;
                G[p][i] = acc;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int p = 0; p < 4; ++p) G[p][i] = 0.f;
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
    u32x4_t bh4[4], bl4[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        u32x4_t kt4, qh4, ql4;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            float kt[2], qt[2], kb[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * wd + e;
                const float eg = fast_exp2(G[p][i]);
                const float egi = fast_exp2(-G[p][i]);
                const float kv = elem(rk[p], i), qv = elem(rq[p], i);
                kt[e] = kv * eg;
                qt[e] = qv * eg;
                kb[e] = kv * egi;
            }
            kt4[wd] = pack2(kt[0], kt[1]);
            uint32_t a, b;
            split2(qt[0], qt[1], a, b); qh4[wd] = a; ql4[wd] = b;
            split2(kb[0], kb[1], a, b); bh4[p][wd] = a; bl4[p][wd] = b;
        }
        const int r = 4 * grp + p;
        *(u32x4_t *)&L.tile[0][tile_off(r, cg)] = kt4;
        *(u32x4_t *)&L.tile[1][tile_off(r, cg)] = qh4;
        *(u32x4_t *)&L.tile[2][tile_off(r, cg)] = ql4;
        *(u32x4_t *)&L.tile[3][tile_off(r, cg)] = bh4[p];
        *(u32x4_t *)&L.tile[4][tile_off(r, cg)] = bl4[p];
    }

    if (grp == 3) {
        // decay over the whole chunk (rows past len contribute nothing)
        f32x4_t g0, g1;
#pragma unroll
        for (int i = 0; i < 4; ++i) { g0[i] = fast_exp2(G[3][i]); g1[i] = fast_exp2(G[3][4 + i]); }
        *(f32x4_t *)&L.gam[8 * cg] = g0;
        *(f32x4_t *)&L.gam[8 * cg + 4] = g1;
        float *gp = (float *)(rec + REC_GAM) + 8 * cg;
        *(f32x4_t *)gp = g0;
        *(f32x4_t *)(gp + 4) = g1;
    }

    __syncthreads();

    // ---- in-chunk products on bf16 MFMA ----------------------------------
    // MFMA view: lane l is row cg (token), k-slots 8grp..8grp+7.
    f32x4_t Akk = {0.f, 0.f, 0.f, 0.f}, AkkT = Akk, AqkT = Akk;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int o = tile_off(cg, 4 * kb + grp);
        const u32x4_t aK = *(const u32x4_t *)&L.tile[0][o];
        const u32x4_t aQh = *(const u32x4_t *)&L.tile[1][o];
        const u32x4_t aQl = *(const u32x4_t *)&L.tile[2][o];
        const u32x4_t aBh = *(const u32x4_t *)&L.tile[3][o];
        const u32x4_t aBl = *(const u32x4_t *)&L.tile[4][o];
        *(u32x4_t *)(rec + REC_KT + (kb * 64 + l) * 16) = aK;
        *(u32x4_t *)(rec + REC_QT + (kb * 64 + l) * 16) = aQh;
        Akk = mfma_k32(aK, aBh, Akk);       // Akk[4grp+j][cg]  = Kt_r . Kb_i
        AkkT = mfma_k32(aBh, aK, AkkT);     // AkkT[4grp+j][cg] = Akk[cg][4grp+j]
        AqkT = mfma_k32(aBh, aQh, AqkT);    // AqkT[4grp+j][cg] = Aqk[cg][4grp+j]
        AqkT = mfma_k32(aBh, aQl, AqkT);
        AqkT = mfma_k32(aBl, aQh, AqkT);
    }
    // channel-major Kb (hi, lo) into tiles 0 and 1: channel 8cg+i, tokens
    // 4grp..4grp+3 (the Gram reads above come first in this wave's LDS order)
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        u32x2_t vh, vl;
        vh[0] = half16(bh4[0][i >> 1], i) | (half16(bh4[1][i >> 1], i) << 16);
        vh[1] = half16(bh4[2][i >> 1], i) | (half16(bh4[3][i >> 1], i) << 16);
        vl[0] = half16(bl4[0][i >> 1], i) | (half16(bl4[1][i >> 1], i) << 16);
        vl[1] = half16(bl4[2][i >> 1], i) | (half16(bl4[3][i >> 1], i) << 16);
        *(u32x2_t *)&L.tile[0][cmaj_off(8 * cg + i, grp)] = vh;
        *(u32x2_t *)&L.tile[1][cmaj_off(8 * cg + i, grp)] = vl;
    }

    // ---- T = (I + L)^{-1}, L = diag(beta) strict_lower(Akk) ---------------
    float br[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) br[j] = L.beta[4 * grp + j];
    const float bc = L.beta[cg];
    f32x4_t N1, N1t, I;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * grp + j;            // accumulator row of this lane
        N1[j] = (cg < r) ? -br[j] * Akk[j] : 0.f;
        N1t[j] = (r < cg) ? -bc * AkkT[j] : 0.f;
        I[j] = (r == cg) ? 1.f : 0.f;
    }
    const f32x4_t P1t = I + N1t;
    const f32x4_t N2 = mm16(N1t, N1), N2t = mm16(N1, N1t);
    const f32x4_t P2 = I + N2;
    const f32x4_t Q12t = mm16(P2, P1t);                 // ((I+N)(I+N^2))^T
    const f32x4_t N4 = mm16(N2t, N2), N4t = mm16(N2, N2t);
    const f32x4_t P4 = I + N4;
    const f32x4_t Q3t = mm16(P4, Q12t);                 // ((I+N)(I+N^2)(I+N^4))^T
    const f32x4_t N8 = mm16(N4t, N4);
    const f32x4_t P8 = I + N8;
    const f32x4_t Tm = mm16(Q3t, P8);                   // T in accumulator layout

    // T diag(beta) in accumulator layout (row 4grp+j, column cg), as (hi, lo):
    // this is also the A-operand layout of (T diag(beta))^T.
    u32x2_t tbh, tbl;
    {
        uint32_t h0, l0, h1, l1;
        split2(Tm[0] * bc, Tm[1] * bc, h0, l0);
        split2(Tm[2] * bc, Tm[3] * bc, h1, l1);
        tbh[0] = h0; tbh[1] = h1; tbl[0] = l0; tbl[1] = l1;
    }
    // masked Aqk^T (i <= r) as (hi, lo) B operand
    float aq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) aq[j] = (4 * grp + j <= cg) ? AqkT[j] : 0.f;
    u32x2_t aqh, aql;
    {
        uint32_t h0, l0, h1, l1;
        split2(aq[0], aq[1], h0, l0);
        split2(aq[2], aq[3], h1, l1);
        aqh[0] = h0; aqh[1] = h1; aql[0] = l0; aql[1] = l1;
    }

    // M^T = (T diag(beta))^T Aqk^T: its accumulator layout is M's A layout.
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    f32x4_t Mt = mfma_k16(tbh, aqh, zero);
    Mt = mfma_k16(tbh, aql, Mt);
    Mt = mfma_k16(tbl, aqh, Mt);
    u32x2_t mo;
    mo[0] = pack2(Mt[0], Mt[1]);
    mo[1] = pack2(Mt[2], Mt[3]);
    *(u32x2_t *)(rec + REC_M + l * 8) = mo;

    __syncthreads();
    // W tiles: W[:, chan(t, .)] = (T diag(beta))^T Kb[:, chan(t, .)] times the
    // chunk decay of that channel; the accumulator layout is the A layout of
    // W^T tile t the scan needs.
#pragma unroll
    for (int tp = 0; tp < 4; ++tp) {
        u32x4_t o;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int ch = state_chan(2 * tp + half, cg);
            const u32x2_t bh = *(const u32x2_t *)&L.tile[0][cmaj_off(ch, grp)];
            const u32x2_t bl = *(const u32x2_t *)&L.tile[1][cmaj_off(ch, grp)];
            f32x4_t Wt = mfma_k16(tbh, bh, zero);
            Wt = mfma_k16(tbh, bl, Wt);
            Wt = mfma_k16(tbl, bh, Wt);
            const float gch = L.gam[ch];
            o[2 * half] = pack2(Wt[0] * gch, Wt[1] * gch);
            o[2 * half + 1] = pack2(Wt[2] * gch, Wt[3] * gch);
        }
        *(u32x4_t *)(rec + REC_WT + (tp * 64 + l) * 16) = o;
    }
}

// One wave per (chunk slot, head): workgroups of one wave, so that the
// 21 KB of LDS a wave needs bounds the occupancy, not a pair of waves.
__global__ __launch_bounds__(64, 2) void intra_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ g, const uint16_t *__restrict__ beta,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float lb2,
    const int32_t *__restrict__ cu, int N, int T, int H, uint8_t *__restrict__ ws)
{
    __shared__ __attribute__((aligned(16))) WaveLds lds;
    const int l = threadIdx.x;
    const int cg = l & 15;
    const int64_t slot = blockIdx.x;
    const int h = blockIdx.y;

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
    if (t0 >= end) return;                         // gap slot, wave-uniform
    const int len = (int)min((int64_t)CS, end - t0);
    uint8_t *rec = ws + ((size_t)slot * H + h) * REC_BYTES;

    const float A = expf(A_log[h]);
    float dtb2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        dtb2[i] = dt_bias ? dt_bias[(size_t)h * HD + 8 * cg + i] * LOG2E : 0.f;

    if (len == CS)
        intra_chunk<true>(lds, q, k, g, beta, A, dtb2, lb2, t0, len, H, h, rec);
    else
        intra_chunk<false>(lds, q, k, g, beta, A, dtb2, lb2, t0, len, H, h, rec);
}

}  // namespace

hipError_t launch_intra(const uint16_t *q, const uint16_t *k, const uint16_t *g,
                        const uint16_t *beta, const float *A_log, const float *dt_bias,
                        float lower_bound, const int32_t *cu, int N, int T, int H,
                        int64_t num_slots, uint8_t *ws, hipStream_t stream)
{
    if (num_slots <= 0) return hipSuccess;
    dim3 grid((unsigned)num_slots, (unsigned)H);
    hipLaunchKernelGGL(intra_kernel, grid, dim3(64), 0, stream,
                       q, k, g, beta, A_log, dt_bias, lower_bound * LOG2E, cu, N, T, H, ws);
    return hipGetLastError();
}

}  // namespace kda
