// Intra-chunk stage, device side: one wave computes the hand-off record of
// one (16-token chunk, head).
//
// Per chunk the wave
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
//   7. writes the record in the register layouts of the scan's MFMA operands.
#pragma once

#include "kda_device.h"

namespace kda {

// LDS scratch of one intra wave: the per-token beta and per-channel chunk
// decay, the two values the wave needs in a layout other than the one it
// computes them in.
template <int KT>
struct WaveLdsT {
    float beta[CS];
    float gam[KT];                  // e^{G_last} per channel
};
using WaveLds = WaveLdsT<HD>;

// Token-per-lane layout: lane l holds token tok = l % 16 and, for each
// 32-channel block kb, the eight channels 32kb + 8(l/16) + i.  For every kb
// this is at once the A and the B operand layout of a 16x16x32 MFMA that
// contracts over channels (row / column = token, k = channel), so the
// in-chunk Gram products and the Kt / Qt records come straight from the
// registers; the cumulative decay over tokens runs across the 16 lanes of a
// DPP row.
// NKB 32-channel blocks: 2, 4 or 8 for head dimension 64, 128 or 256.
template <int NKB>
struct IntraInT {
    u32x4_t g[NKB], q[NKB], k[NKB]; // [kb]: 8 bf16 channels of this lane's token
    uint32_t beta;                  // logit of this lane's token
    uint32_t gs;                    // scalar gate of this lane's token (SG form)
};
using IntraIn = IntraInT<4>;

template <bool SG, int KT = HD>
__device__ __forceinline__ void intra_load(IntraInT<KT / 32> &in, const uint16_t *__restrict__ q,
                                           const uint16_t *__restrict__ k,
                                           const uint16_t *__restrict__ g,
                                           const uint16_t *__restrict__ beta,
                                           int64_t t0, int len, int H, int hh, int K) {
    // K = KT, or K = 64 on KT = 128: channels from K on are zeros (zero keys and queries add
    // nothing to the in-chunk products, the W rows or the state)
    const int l = threadIdx.x & 63;
    const int tok = l & 15, cgp = l >> 4;
    const size_t row_elems = (size_t)H * K;
    const size_t base = ((size_t)t0 * H + hh) * K;
    const uint32_t bytes = len > 0 ? (uint32_t)(((size_t)(len - 1) * row_elems + K) * 2) : 0u;
    const __amdgpu_buffer_rsrc_t sg = make_rsrc(g + base, bytes);
    const __amdgpu_buffer_rsrc_t sq = make_rsrc(q + base, bytes);
    const __amdgpu_buffer_rsrc_t sk = make_rsrc(k + base, bytes);
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int kb = 0; kb < KT / 32; ++kb) {
        const int off = (int)((tok * row_elems + 32 * kb + 8 * cgp) * 2);
        in.g[kb] = in.q[kb] = in.k[kb] = z;
        if (32 * kb < K) {                          // block-uniform
            if (!SG)
                in.g[kb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sg, off, 0, 0));
            in.q[kb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sq, off, 0, 0));
            in.k[kb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sk, off, 0, 0));
        }
    }
    // beta (and the scalar gate of the SG form) are [token, head]
    const uint32_t tb = len > 0 ? (uint32_t)(((size_t)(len - 1) * H + 1) * 2) : 0u;
    const __amdgpu_buffer_rsrc_t sb = make_rsrc(beta + (size_t)t0 * H + hh, tb);
    in.beta = __builtin_amdgcn_raw_buffer_load_b16(sb, tok * H * 2, 0, 0);
    if (SG) {
        const __amdgpu_buffer_rsrc_t ss = make_rsrc(g + (size_t)t0 * H + hh, tb);
        in.gs = __builtin_amdgcn_raw_buffer_load_b16(ss, tok * H * 2, 0, 0);
    }
}

// dt_bias of one head in log2 units into LDS (KT floats; zeros when absent
// and for channels from K on), by the lanes of the calling wave.  SG form: dt_bias is [H], one value per
// head, staged into dtb_lds[0].
template <bool SG = false, int KT = HD>
__device__ __forceinline__ void stage_dtb(float *__restrict__ dtb_lds, const float *__restrict__ dt_bias,
                                          int hh, int K = HD) {
    const int l = threadIdx.x & 63;
    if (SG) {
        if (l == 0) dtb_lds[0] = dt_bias ? dt_bias[hh] * LOG2E : 0.f;
        return;
    }
#pragma unroll
    for (int r = 0; r < KT / 64; ++r) {
        const int c = 64 * r + l;
        dtb_lds[c] = (dt_bias && c < K) ? dt_bias[(size_t)hh * K + c] * LOG2E : 0.f;
    }
}

// Inclusive prefix sum over the 16 lanes of each DPP row (lanes past the
// row start read 0 through bound_ctrl).
template <int SH>
__device__ __forceinline__ float row_shr(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x110 + SH, 0xf, 0xf, true));
}
// Eight independent prefix sums, interleaved step by step.
__device__ __forceinline__ void row_prefix8(float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] += row_shr<1>(x[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] += row_shr<2>(x[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] += row_shr<4>(x[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] += row_shr<8>(x[i]);
}

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

// beta = sigmoid(logit) of one token, the logit a bf16 word.
__device__ __forceinline__ float beta_sigmoid(uint32_t logit) {
    const float x = bf16f((uint16_t)logit);
    return __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * LOG2E));
}

// The gate of the lane's token on the eight channels 32kb + 8grp + i of
// g8 (bf16 pre-activation gate values), in base 2:
//   log2 alpha = max(-A log2(1 + 2^{x2}), lb2),  x2 = g log2 e + dt_bias log2 e,
// zero for a token past the chunk's length (live false), then the
// inclusive cumulative sum over the chunk's tokens, which are the 16 lanes
// of a DPP row.  dtb_lds: the head's dt_bias in log2 units.
__device__ __forceinline__ void gate_cumsum(float (&G)[8], const u32x4_t &g8,
                                            const float *__restrict__ dtb_lds, int kb, int grp,
                                            float A, float lb2, bool live) {
    float dtb2[8];
    *(f32x4_t *)&dtb2[0] = *(const f32x4_t *)&dtb_lds[32 * kb + 8 * grp];
    *(f32x4_t *)&dtb2[4] = *(const f32x4_t *)&dtb_lds[32 * kb + 8 * grp + 4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x2 = elem(g8, i) * LOG2E + dtb2[i];
        const float u = fast_log2(1.f + fast_exp2(x2));
        const float la = fmaxf(-A * u, lb2);
        G[i] = live ? la : 0.f;
    }
    row_prefix8(G);
}

// One (chunk, head) by one wave, inputs in the token-per-lane layout.
// FULL: all 16 rows are tokens of the sequence (no masking of the
// cumulative decay).  SG: the Gated DeltaNet form, one gate value per
// (token, head) for all channels (in.gs, dt_bias in dtb_lds[0]); the gate
// and its cumulative sum are then computed once per token with the same
// operations as in the per-channel form, so the results equal the
// per-channel form's on inputs broadcast over channels, bit for bit.
// dtb_lds: the head's dt_bias in log2 units (LDS).  `rec` is the record in
// global memory.  KT: key channels of the tiles (128, or 256 for head
// dimension 256: eight channel blocks, sixteen state row tiles).
template <bool FULL, bool SG = false, int KT = HD>
__device__ __forceinline__ void intra_compute(WaveLdsT<KT> &L, const IntraInT<KT / 32> &in, float A,
                                              const float *__restrict__ dtb_lds, float lb2, int len,
                                              uint8_t *__restrict__ rec) {
    typedef RecLayout<KT> R;
    constexpr int NKB = KT / 32;
    const int l = threadIdx.x & 63;
    const int tok = l & 15;        // token of this lane (operand view)
    const int grp = l >> 4;        // accumulator view: rows 4grp .. 4grp+3, column tok
    const int cg = tok;
    const bool live = FULL || tok < len;

    {
        const float b = beta_sigmoid(in.beta);
        if (grp == 0) L.beta[tok] = live ? b : 0.f;
    }

    // Identity as a 16x16x16 B operand (lane l: k = 4(l/16) + j, column l%16):
    // D = X I moves X from the A-operand layout (one row, four k per lane)
    // to the accumulator layout (four rows, one column per lane), i.e. it
    // transposes the lane / register roles of a 16x16 tile exactly.
    u32x2_t eye;
    {
        const uint32_t one = 0x3f80u;           // bf16 1.0
        const int d = tok - 4 * grp;            // which j of this lane is on the diagonal
        eye[0] = (d == 0 ? one : 0u) | (d == 1 ? one << 16 : 0u);
        eye[1] = (d == 2 ? one : 0u) | (d == 3 ? one << 16 : 0u);
    }
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

    // ---- per 32-channel block: gate, cumulative decay, operands, Grams -----
    // Akk[r][i] = Kt_r . Kb_i, AkkT its transpose, AqkT[i][r] = Qt_r . Kb_i
    // (fp32-accurate from hi/lo parts); Kb hi/lo also transposed into the
    // B-operand layout of the W products (kbh/kbl[t], state row tile t).
    f32x4_t Akk = zero, AkkT = zero, AqkT = zero;
    u32x2_t kbh[2 * NKB], kbl[2 * NKB];
    float Gs = 0.f;                                  // SG form: the one cumulative gate
    if (SG && A > 0.f) {
        const float x2 = bf16f((uint16_t)in.gs) * LOG2E + dtb_lds[0];
        const float u = fast_log2(1.f + fast_exp2(x2));
        const float la = fmaxf(-A * u, lb2);
        Gs = live ? la : 0.f;
        Gs += row_shr<1>(Gs);
        Gs += row_shr<2>(Gs);
        Gs += row_shr<4>(Gs);
        Gs += row_shr<8>(Gs);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        float G[8];
        if (SG) {
#pragma unroll
            for (int i = 0; i < 8; ++i) G[i] = Gs;
        } else if (A > 0.f) {
            gate_cumsum(G, in.g[kb], dtb_lds, kb, grp, A, lb2, live);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) G[i] = 0.f;
        }
        u32x4_t kt4, qh4, ql4, bh4, bl4;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            float kt[2], qt[2], kbv[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * wd + e;
                const float eg = fast_exp2(G[i]);
                const float egi = fast_exp2(-G[i]);
                const float kv = elem(in.k[kb], i), qv = elem(in.q[kb], i);
                kt[e] = kv * eg;
                qt[e] = qv * eg;
                kbv[e] = kv * egi;
            }
            kt4[wd] = pack2(kt[0], kt[1]);
            uint32_t a, b;
            split2(qt[0], qt[1], a, b); qh4[wd] = a; ql4[wd] = b;
            split2(kbv[0], kbv[1], a, b); bh4[wd] = a; bl4[wd] = b;
        }
        // chunk decay per channel: the token-15 lanes hold G at the last row
        // (rows past len added nothing)
        if (tok == CS - 1) {
            f32x4_t g0, g1;
#pragma unroll
            for (int i = 0; i < 4; ++i) { g0[i] = fast_exp2(G[i]); g1[i] = fast_exp2(G[4 + i]); }
            const int ch = 32 * kb + 8 * grp;
            *(f32x4_t *)&L.gam[ch] = g0;
            *(f32x4_t *)&L.gam[ch + 4] = g1;
        }
        // records are written with non-temporal stores (see intra_kernel)
        __builtin_nontemporal_store(kt4, (u32x4_t *)(rec + R::KTO + (kb * 64 + l) * 16));
        __builtin_nontemporal_store(qh4, (u32x4_t *)(rec + R::QT + (kb * 64 + l) * 16));
        Akk = mfma_k32(kt4, bh4, Akk);          // Akk[4grp+j][cg]  = Kt_r . Kb_i
        AkkT = mfma_k32(bh4, kt4, AkkT);        // AkkT[4grp+j][cg] = Akk[cg][4grp+j]
        AqkT = mfma_k32(bh4, qh4, AqkT);        // AqkT[4grp+j][cg] = Aqk[cg][4grp+j]
        AqkT = mfma_k32(bh4, ql4, AqkT);
        AqkT = mfma_k32(bl4, qh4, AqkT);
        // state row tiles t = 2kb + h hold channels 32kb + 8(l/16) + 4h + j:
        // words 2h, 2h+1 of this block are their A operands.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x2_t ah = {bh4[2 * h], bh4[2 * h + 1]}, al = {bl4[2 * h], bl4[2 * h + 1]};
            const f32x4_t dh = mfma_k16(ah, eye, zero);
            const f32x4_t dl = mfma_k16(al, eye, zero);
            kbh[2 * kb + h] = {pack2(dh[0], dh[1]), pack2(dh[2], dh[3])};   // exact: bf16 values
            kbl[2 * kb + h] = {pack2(dl[0], dl[1]), pack2(dl[2], dl[3])};
        }
    }

    wave_lds_sync();
    // the chunk decay into the record from LDS in one coalesced store (four
    // lanes' 16-byte pieces per block cost several times as much)
    if constexpr (KT == 64) {
        __builtin_nontemporal_store(*(const uint32_t *)&L.gam[l], (uint32_t *)(rec + R::GAM + l * 4));
    } else {
#pragma unroll
        for (int p = 0; p < KT / 128; ++p)
            __builtin_nontemporal_store(*(const u32x2_t *)&L.gam[2 * (64 * p + l)], (u32x2_t *)(rec + R::GAM + (64 * p + l) * 8));
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
    f32x4_t Mt = mfma_k16(tbh, aqh, zero);
    Mt = mfma_k16(tbh, aql, Mt);
    Mt = mfma_k16(tbl, aqh, Mt);
    u32x2_t mo;
    mo[0] = pack2(Mt[0], Mt[1]);
    mo[1] = pack2(Mt[2], Mt[3]);
    __builtin_nontemporal_store(mo, (u32x2_t *)(rec + R::M + l * 8));

    // W tiles: W[:, chan(t, .)] = (T diag(beta))^T Kb[:, chan(t, .)] times the
    // chunk decay of that channel; the accumulator layout is the A layout of
    // W^T tile t the scan needs.
#pragma unroll
    for (int tp = 0; tp < NKB; ++tp) {
        u32x4_t o;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int t = 2 * tp + half;
            f32x4_t Wt = mfma_k16(tbh, kbh[t], zero);
            Wt = mfma_k16(tbh, kbl[t], Wt);
            Wt = mfma_k16(tbl, kbh[t], Wt);
            const float gch = L.gam[state_chan(t, cg)];
            o[2 * half] = pack2(Wt[0] * gch, Wt[1] * gch);
            o[2 * half + 1] = pack2(Wt[2] * gch, Wt[3] * gch);
        }
        __builtin_nontemporal_store(o, (u32x4_t *)(rec + R::WT + (tp * 64 + l) * 16));
    }
}

}  // namespace kda
