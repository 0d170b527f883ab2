// Chunk of 32 tokens: the intra-chunk stage (one wave per (chunk, head))
// and the scan's per-chunk step, device side.
//
// Per chunk of up to 32 tokens with incoming state S0 (per head):
//   G_r  = inclusive cumulative log2-decay over the chunk, per channel
//   Kt   = k 2^{G},  Qt = q 2^{G}                                   (32 x 128)
//   Khat = k 2^{G_last - G}                                          (32 x 128)
//   A[r][i]   = sum_c k_r k_i 2^{G_r - G_i}   (i < r),  L = diag(beta) A
//   Aqk[r][i] = sum_c q_r k_i 2^{G_r - G_i}   (i <= r)
//   T  = (I + L)^{-1},  Tb = T diag(beta)
//   M  = Aqk Tb,   W = Tb^T Khat                                      (intra stage)
//   X  = V - Kt S0,  O = scale (Qt S0 + M X),  S = diag(2^{G_last}) S0 + W^T X  (scan)
// This is the chunkwise ("specialized DPLR") algorithm the FlashKDA write-up
// credits for KDA's efficiency ("Moonshot AI Open-Sources FlashKDA",
// section "Why KDA?"), at twice the chunk length of its section "What
// makes the kernel fast": on gfx950 the scan's pace is set by its chain of
// dependent chunk steps, and 32-token chunks halve their number while each
// step still fits the 16x16x32 MFMA tiles.
//
// Range.  2^{G_r - G_i} is formed as a product of two factors inside each
// 16-token sub-block b (rows 16b .. 16b+15), with g^b the cumulative decay
// from the sub-block's start and Gam_b its total:
//   r, i in sub-block b:     2^{g^b_r} * 2^{-g^b_i}            (F^b, B^b)
//   r in 1, i in 0:          2^{g^1_r} * 2^{Gam_0 - g^0_i}     (F^1, e^0)
// Only the diagonal blocks have a factor above 1 (at most 2^{16 |lb| log2 e}),
// so the lower bound range is that of a 16-token chunk; every other factor
// is at most 1.  Kt, Qt, Khat and the chunk decay are products of factors
// at most 1 (they may only underflow, where the true value is negligible).
//
// The triangular inverse is blockwise over the 16 x 16 blocks:
//   T00 = (I + L00)^{-1},  T11 = (I + L11)^{-1},  T10 = -T11 L10 T00,
// each diagonal block by the product form of the Neumann series on fp32
// 16x16x4 MFMAs (the small-inverse step of the same section).
#pragma once

#include "kda_intra_dev.h"

namespace kda {

constexpr int C32 = 32;                    // tokens per chunk

// Hand-off record of one (32-token chunk slot, head), in the register
// layouts of the scan's MFMA operands (16x16x32 bf16):
//   KT  [kb 0..3][rt 0..1][lane][8 bf16]  Kt rows 16rt + l%16, channels
//        32kb + 8(l/16) + i (A operand of P = Kt S0)
//   QT  same for Qt
//   WT  [t 0..7][lane][8 bf16]  W^T state-row tile t (rows chan(t, l%16))
//        as an A operand whose k index 8(l/16) + i stands for token
//        tau(8(l/16) + i) = 4(l/16) + i (i < 4), 16 + 4(l/16) + i - 4 (i >= 4)
//   M   [rt 0..1][lane][8 bf16]  M rows 16rt + l%16, k as in WT
//   GAM [128 fp32]  2^{G_last} per channel
// The k order tau is the order in which the accumulators of the two token
// row tiles of X = V - Kt S0 hold their rows, so X feeds the update and
// M X without moving.
struct Rec32 {
    static constexpr int KT = 0;
    static constexpr int QT = 8192;
    static constexpr int WT = 16384;
    static constexpr int M = 24576;
    static constexpr int GAM = 26624;
    static constexpr int BYTES = 27648;      // 27 one-kilobyte units
};

__host__ __device__ constexpr int64_t c32_slot0_of(int64_t start, int n) { return start / C32 + n; }

// First chunk slot of sequence n: floor(start / 32) + n.  Slots of
// consecutive sequences never overlap and all lie below floor(total/32) + N.
__device__ __forceinline__ int64_t seq_slot0_32(const int32_t *cu, int n, int T) {
    const int64_t s = cu ? (int64_t)cu[n] : (int64_t)n * T;
    return c32_slot0_of(s, n);
}

struct Wave32Lds {
    float beta[C32];
    float gam[HD];
};
// Khat of sub-block b, state row tile t, as bf16 B operands of the W
// products, [b][t][lane], held between the channel-block loop and the W
// products.  W is stored in bf16 and Khat enters it through one product, so
// Khat's own bf16 rounding adds no more than the record's.
struct Khat32Lds {
    u32x2_t khat[2][8][64];
};

// Token-per-lane inputs of one 32-token chunk: lane l holds tokens l%16
// (sub-block 0) and 16 + l%16 (sub-block 1), eight channels 32kb + 8(l/16) + i
// of a 32-channel block kb.  The wave reads one block at a time, one block
// ahead of its use.
struct Intra32Src {
    __amdgpu_buffer_rsrc_t g, q, k;
    int row_bytes;                     // bytes between consecutive token rows
    int K;
    uint32_t beta[2];
    uint32_t gs[2];                    // scalar gate (Gated DeltaNet form)
};
struct Intra32Blk {
    u32x4_t g[2], q[2], k[2];
};

// Sets up the reads of one chunk of len tokens starting at token row t0
// (K = 128, or 64 with the channels from 64 on read as zeros) and reads the
// per-token values.  Rows past len read as zeros.
template <bool SG>
__device__ __forceinline__ void intra32_src(Intra32Src &s, const uint16_t *__restrict__ q,
                                            const uint16_t *__restrict__ k,
                                            const uint16_t *__restrict__ g,
                                            const uint16_t *__restrict__ beta, int64_t t0,
                                            int len, int H, int hh, int K) {
    const int l = threadIdx.x & 63;
    const int tok = l & 15;
    const size_t row_elems = (size_t)H * K;
    const size_t base = ((size_t)t0 * H + hh) * K;
    const uint32_t bytes = len > 0 ? (uint32_t)(((size_t)(len - 1) * row_elems + K) * 2) : 0u;
    s.g = make_rsrc(g + base, SG ? 0u : bytes);
    s.q = make_rsrc(q + base, bytes);
    s.k = make_rsrc(k + base, bytes);
    s.row_bytes = (int)(row_elems * 2);
    s.K = K;
    const uint32_t tb = len > 0 ? (uint32_t)(((size_t)(len - 1) * H + 1) * 2) : 0u;
    const __amdgpu_buffer_rsrc_t sb = make_rsrc(beta + (size_t)t0 * H + hh, tb);
#pragma unroll
    for (int b = 0; b < 2; ++b)
        s.beta[b] = __builtin_amdgcn_raw_buffer_load_b16(sb, (16 * b + tok) * H * 2, 0, 0);
    if (SG) {
        const __amdgpu_buffer_rsrc_t ss = make_rsrc(g + (size_t)t0 * H + hh, tb);
#pragma unroll
        for (int b = 0; b < 2; ++b)
            s.gs[b] = __builtin_amdgcn_raw_buffer_load_b16(ss, (16 * b + tok) * H * 2, 0, 0);
    } else {
        s.gs[0] = s.gs[1] = 0u;
    }
}

template <bool SG>
__device__ __forceinline__ void intra32_read(Intra32Blk &x, const Intra32Src &s, int kb) {
    const int l = threadIdx.x & 63;
    const int tok = l & 15, cgp = l >> 4;
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int off = (16 * b + tok) * s.row_bytes + (32 * kb + 8 * cgp) * 2;
        x.g[b] = x.q[b] = x.k[b] = z;
        if (32 * kb < s.K) {                    // uniform
            if (!SG) x.g[b] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(s.g, off, 0, 0));
            x.q[b] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(s.q, off, 0, 0));
            x.k[b] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(s.k, off, 0, 0));
        }
    }
}

// Lane 15 of each 16-lane row, broadcast to the row (DPP row_newbcast).
__device__ __forceinline__ float row_last(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                              0x15f, 0xf, 0xf, true));
}

// The Neumann product inverse of one 16x16 unit-lower-triangular block
// (I - N)^{-1} = (I + N)(I + N^2)(I + N^4)(I + N^8) with N = -L strictly
// lower: n1 / n1t are the accumulator layouts of N and N^T.  Returns T and
// T^T in accumulator layout (the factors commute).
__device__ __forceinline__ void neumann16(const f32x4_t &n1, const f32x4_t &n1t, const f32x4_t &eye4,
                                          f32x4_t &t, f32x4_t &tt) {
    const f32x4_t p1t = eye4 + n1t;
    const f32x4_t n2 = mm16(n1t, n1), n2t = mm16(n1, n1t);
    const f32x4_t p2 = eye4 + n2;
    const f32x4_t q12t = mm16(p2, p1t);                 // ((I+N)(I+N^2))^T
    const f32x4_t n4 = mm16(n2t, n2), n4t = mm16(n2, n2t);
    const f32x4_t p4 = eye4 + n4;
    const f32x4_t q3t = mm16(p4, q12t);                 // ((I+N)(I+N^2)(I+N^4))^T
    const f32x4_t n8 = mm16(n4t, n4);
    const f32x4_t p8 = eye4 + n8;
    t = mm16(q3t, p8);                                   // Q3 P8
    tt = mm16(p8, q3t);                                  // P8^T Q3^T = (Q3 P8)^T
}

__device__ __forceinline__ void split2v(const f32x4_t &x, float s, u32x2_t &hi, u32x2_t &lo) {
    uint32_t h0, l0, h1, l1;
    split2(x[0] * s, x[1] * s, h0, l0);
    split2(x[2] * s, x[3] * s, h1, l1);
    hi[0] = h0; hi[1] = h1; lo[0] = l0; lo[1] = l1;
}

// a_hi a + a_hi b_lo + a_lo b_hi for 16x16x16 bf16 operands: an fp32-accurate
// product of (hi, lo) pairs, accumulated onto c.
__device__ __forceinline__ f32x4_t mfma3_k16(u32x2_t ah, u32x2_t al, u32x2_t bh, u32x2_t bl, f32x4_t c) {
    c = mfma_k16(ah, bh, c);
    c = mfma_k16(ah, bl, c);
    return mfma_k16(al, bh, c);
}

// One (32-token chunk, head) by one wave.  FULL: all 32 rows are tokens of
// the sequence.  SG: the Gated DeltaNet form (one gate value per token and
// head, dt_bias in dtb_lds[0]), computed once per token with the same
// operations as the per-channel form, so results equal the per-channel
// form's on broadcast inputs bit for bit.  `rec`: the record (global
// memory, or any address space the stores reach).  NT: non-temporal record
// stores.
// PREFETCH: read the next channel block's inputs while computing this one
// (more registers, fewer exposed load latencies).
template <bool FULL, bool SG, bool NT = true, bool PREFETCH = true>
__device__ __forceinline__ void intra32_compute(Wave32Lds &L, Khat32Lds *KL, const Intra32Src &in,
                                                float A, const float *__restrict__ dtb_lds, float lb2,
                                                int len, uint8_t *__restrict__ rec) {
    typedef Rec32 R;
    const int l = threadIdx.x & 63;
    const int tok = l & 15, grp = l >> 4, cg = tok;
    bool live[2];
    live[0] = FULL || tok < len;
    live[1] = FULL || 16 + tok < len;
    auto st16 = [&](const u32x4_t &v, int off) {
        if (NT) __builtin_nontemporal_store(v, (u32x4_t *)(rec + off));
        else *(u32x4_t *)(rec + off) = v;
    };

#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const float x = bf16f((uint16_t)in.beta[b]);
        const float bv = __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * LOG2E));
        if (grp == 0) L.beta[16 * b + tok] = live[b] ? bv : 0.f;
    }
    u32x2_t eye;
    {
        const uint32_t one = 0x3f80u;
        const int d = tok - 4 * grp;
        eye[0] = (d == 0 ? one : 0u) | (d == 1 ? one << 16 : 0u);
        eye[1] = (d == 2 ? one : 0u) | (d == 3 ? one << 16 : 0u);
    }
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

    // Gram blocks: Akk rows / cols by sub-block (A10: rows in 1, columns in
    // 0), AkkT the transposes of the diagonal ones, AqkT[i][r] = Aqk[r][i].
    f32x4_t A00 = zero, A00t = zero, A11 = zero, A11t = zero, A10 = zero;
    f32x4_t Q00t = zero, Q11t = zero, Q10t = zero;

    // Khat of sub-block b, channel block kb (token-per-lane words) into the
    // B layout of the W products through the identity (exact for bf16
    // values), staged in LDS until the W products
    auto stage_khat = [&](int b, int kb, const u32x4_t &kht) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x2_t ah = {kht[2 * h], kht[2 * h + 1]};
            const f32x4_t dh = mfma_k16(ah, eye, zero);
            KL->khat[b][2 * kb + h][l] = {pack2(dh[0], dh[1]), pack2(dh[2], dh[3])};
        }
    };

    float gsc[2] = {0.f, 0.f};         // SG form: the cumulative gate of each sub-block
    if (SG && A > 0.f) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const float x2 = bf16f((uint16_t)in.gs[b]) * LOG2E + dtb_lds[0];
            const float u = fast_log2(1.f + fast_exp2(x2));
            const float la = fmaxf(-A * u, lb2);
            float s = live[b] ? la : 0.f;
            s += row_shr<1>(s);
            s += row_shr<2>(s);
            s += row_shr<4>(s);
            s += row_shr<8>(s);
            gsc[b] = s;
        }
    }
    Intra32Blk nxt;
    if (PREFETCH) intra32_read<SG>(nxt, in, 0);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        Intra32Blk cur;
        if (PREFETCH) {
            cur = nxt;
            if (kb + 1 < 4) intra32_read<SG>(nxt, in, kb + 1);
        } else {
            intra32_read<SG>(cur, in, kb);
        }
        float gl[2][8];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if (SG) {
#pragma unroll
                for (int i = 0; i < 8; ++i) gl[b][i] = gsc[b];
            } else if (A > 0.f) {
                float dtb2[8];
                *(f32x4_t *)&dtb2[0] = *(const f32x4_t *)&dtb_lds[32 * kb + 8 * grp];
                *(f32x4_t *)&dtb2[4] = *(const f32x4_t *)&dtb_lds[32 * kb + 8 * grp + 4];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float x2 = elem(cur.g[b], i) * LOG2E + dtb2[i];
                    const float u = fast_log2(1.f + fast_exp2(x2));
                    const float la = fmaxf(-A * u, lb2);
                    gl[b][i] = live[b] ? la : 0.f;
                }
                row_prefix8(gl[b]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) gl[b][i] = 0.f;
            }
        }
        // per channel: F = 2^{g}, Bv = 2^{-g}, eg = 2^{Gam} (F at the
        // sub-block's last row), e = 2^{Gam - g}.  Sub-block 1 first, its
        // products issued before sub-block 0's operands exist, so that only
        // its Kt / Qt pieces stay live for the off-diagonal block.
        float F0[8], eg0[8], eg1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            F0[i] = fast_exp2(gl[0][i]);
            eg0[i] = row_last(F0[i]);
        }
        u32x4_t kf1, qfh1, qfl1;
        {
            u32x4_t kbh1, kbl1, kt1, qt1, kht1;
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
                float kF[2], qF[2], kB[2], kt[2], qt[2], kh[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int i = 2 * wd + e;
                    const float F = fast_exp2(gl[1][i]);
                    const float Bv = fast_exp2(-gl[1][i]);
                    eg1[i] = row_last(F);
                    const float kv = elem(cur.k[1], i), qv = elem(cur.q[1], i);
                    kF[e] = kv * F;
                    qF[e] = qv * F;
                    kB[e] = kv * Bv;
                    kt[e] = kF[e] * eg0[i];              // chunk-level Kt, Qt of sub-block 1
                    qt[e] = qF[e] * eg0[i];
                    kh[e] = kv * (Bv * eg1[i]);          // k 2^{G_last - G} = k 2^{Gam_1 - g^1}
                }
                uint32_t h, lo;
                kf1[wd] = pack2(kF[0], kF[1]);
                split2(kB[0], kB[1], h, lo); kbh1[wd] = h; kbl1[wd] = lo;
                split2(qF[0], qF[1], h, lo); qfh1[wd] = h; qfl1[wd] = lo;
                kht1[wd] = pack2(kh[0], kh[1]);
                kt1[wd] = pack2(kt[0], kt[1]);
                qt1[wd] = pack2(qt[0], qt[1]);
            }
            st16(kt1, R::KT + ((kb * 2 + 1) * 64 + l) * 16);
            st16(qt1, R::QT + ((kb * 2 + 1) * 64 + l) * 16);
            A11 = mfma_k32(kf1, kbh1, A11);
            A11t = mfma_k32(kbh1, kf1, A11t);
            Q11t = mfma_k32(kbh1, qfh1, Q11t);
            Q11t = mfma_k32(kbh1, qfl1, Q11t);
            Q11t = mfma_k32(kbl1, qfh1, Q11t);
            stage_khat(1, kb, kht1);
        }
        {
            u32x4_t kf0, kbh0, kbl0, qfh0, qfl0, ke0h, ke0l, kht0;
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
                float kF[2], qF[2], kB[2], ke[2], kh[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int i = 2 * wd + e;
                    const float Bv = fast_exp2(-gl[0][i]);
                    const float kv = elem(cur.k[0], i), qv = elem(cur.q[0], i);
                    kF[e] = kv * F0[i];
                    qF[e] = qv * F0[i];
                    kB[e] = kv * Bv;
                    ke[e] = kv * (Bv * eg0[i]);          // k 2^{Gam_0 - g^0}
                    kh[e] = ke[e] * eg1[i];              // k 2^{G_last - G}
                }
                uint32_t h, lo;
                kf0[wd] = pack2(kF[0], kF[1]);
                split2(kB[0], kB[1], h, lo); kbh0[wd] = h; kbl0[wd] = lo;
                split2(qF[0], qF[1], h, lo); qfh0[wd] = h; qfl0[wd] = lo;
                split2(ke[0], ke[1], h, lo); ke0h[wd] = h; ke0l[wd] = lo;
                kht0[wd] = pack2(kh[0], kh[1]);
            }
            // sub-block 0: the local factors are the chunk-level ones (Qt's
            // record is its hi part)
            st16(kf0, R::KT + ((kb * 2 + 0) * 64 + l) * 16);
            st16(qfh0, R::QT + ((kb * 2 + 0) * 64 + l) * 16);
            A00 = mfma_k32(kf0, kbh0, A00);
            A00t = mfma_k32(kbh0, kf0, A00t);
            A10 = mfma_k32(kf1, ke0h, A10);
            Q00t = mfma_k32(kbh0, qfh0, Q00t);
            Q00t = mfma_k32(kbh0, qfl0, Q00t);
            Q00t = mfma_k32(kbl0, qfh0, Q00t);
            Q10t = mfma_k32(ke0h, qfh1, Q10t);
            Q10t = mfma_k32(ke0h, qfl1, Q10t);
            Q10t = mfma_k32(ke0l, qfh1, Q10t);
            stage_khat(0, kb, kht0);
        }
        // chunk decay per channel: 2^{Gam_0 + Gam_1}
        if (tok == 15) {
            f32x4_t g0, g1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                g0[i] = eg0[i] * eg1[i];
                g1[i] = eg0[4 + i] * eg1[4 + i];
            }
            const int ch = 32 * kb + 8 * grp;
            *(f32x4_t *)&L.gam[ch] = g0;
            *(f32x4_t *)&L.gam[ch + 4] = g1;
        }
    }

    wave_lds_sync();
    {
        const u32x2_t gw = *(const u32x2_t *)&L.gam[2 * l];
        if (NT) __builtin_nontemporal_store(gw, (u32x2_t *)(rec + R::GAM + l * 8));
        else *(u32x2_t *)(rec + R::GAM + l * 8) = gw;
    }

    // ---- blockwise inverse -------------------------------------------------
    float br[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) { br[0][j] = L.beta[4 * grp + j]; br[1][j] = L.beta[16 + 4 * grp + j]; }
    const float bc0 = L.beta[cg], bc1 = L.beta[16 + cg];
    f32x4_t I4;
    f32x4_t n0, n0t, n1, n1t, l10;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * grp + j;
        n0[j] = (cg < r) ? -br[0][j] * A00[j] : 0.f;
        n0t[j] = (r < cg) ? -bc0 * A00t[j] : 0.f;
        n1[j] = (cg < r) ? -br[1][j] * A11[j] : 0.f;
        n1t[j] = (r < cg) ? -bc1 * A11t[j] : 0.f;
        l10[j] = br[1][j] * A10[j];
        I4[j] = (r == cg) ? 1.f : 0.f;
    }
    f32x4_t T00, T00t, T11, T11t;
    neumann16(n0, n0t, I4, T00, T00t);
    neumann16(n1, n1t, I4, T11, T11t);
    const f32x4_t Ut = mm16(l10, T11t);                // (T11 L10)^T = L10^T T11^T
    const f32x4_t T10 = -mm16(Ut, T00);                // -T11 L10 T00

    // T diag(beta) blocks as (hi, lo) A operands of the transposed products
    u32x2_t tb00h, tb00l, tb11h, tb11l, tb10h, tb10l;
    split2v(T00, bc0, tb00h, tb00l);
    split2v(T11, bc1, tb11h, tb11l);
    split2v(T10, bc0, tb10h, tb10l);

    // ---- M^T blocks: M = Aqk T diag(beta) ------------------------------------
    f32x4_t a00, a11;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a00[j] = (4 * grp + j <= cg) ? Q00t[j] : 0.f;
        a11[j] = (4 * grp + j <= cg) ? Q11t[j] : 0.f;
    }
    u32x2_t q00h, q00l, q11h, q11l, q10h, q10l;
    split2v(a00, 1.f, q00h, q00l);
    split2v(a11, 1.f, q11h, q11l);
    split2v(Q10t, 1.f, q10h, q10l);
    const f32x4_t M00t = mfma3_k16(tb00h, tb00l, q00h, q00l, zero);
    const f32x4_t M11t = mfma3_k16(tb11h, tb11l, q11h, q11l, zero);
    f32x4_t M10t = mfma3_k16(tb00h, tb00l, q10h, q10l, zero);
    M10t = mfma3_k16(tb10h, tb10l, q11h, q11l, M10t);
    {
        const u32x4_t m0 = {pack2(M00t[0], M00t[1]), pack2(M00t[2], M00t[3]), 0u, 0u};
        const u32x4_t m1 = {pack2(M10t[0], M10t[1]), pack2(M10t[2], M10t[3]),
                            pack2(M11t[0], M11t[1]), pack2(M11t[2], M11t[3])};
        st16(m0, R::M + l * 16);
        st16(m1, R::M + (64 + l) * 16);
    }

    // ---- W tiles: W = Tb^T Khat ---------------------------------------------
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const u32x2_t k0 = KL->khat[0][t][l], k1 = KL->khat[1][t][l];
        f32x4_t w0 = mfma_k16(tb00h, k0, zero);
        w0 = mfma_k16(tb00l, k0, w0);
        w0 = mfma_k16(tb10h, k1, w0);
        w0 = mfma_k16(tb10l, k1, w0);
        f32x4_t w1 = mfma_k16(tb11h, k1, zero);
        w1 = mfma_k16(tb11l, k1, w1);
        const u32x4_t o = {pack2(w0[0], w0[1]), pack2(w0[2], w0[3]), pack2(w1[0], w1[1]),
                           pack2(w1[2], w1[3])};
        st16(o, R::WT + (t * 64 + l) * 16);
    }
}

}  // namespace kda
