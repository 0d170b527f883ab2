// Intra-chunk stage of one 32-token chunk by a team of four waves, one per
// 32-channel block kb (the record layout and the arithmetic are those of
// kda_c32_dev.h).  Splitting the chunk over four waves (on four SIMDs)
// shortens the time from a chunk's inputs to its record about fourfold,
// which is what lets producers run only a few chunks ahead of the scan that
// consumes their records.
//
//   phase 1 (each wave, its channel block): gate, cumulative decays, the
//            decayed operands, the Kt / Qt record pieces, the chunk decay of
//            its channels, its Khat tiles (kept in registers), and its
//            partial Gram tiles A00, A11, A10, Aqk00^T, Aqk11^T, Aqk10^T,
//            written to LDS;
//   phase 2 (wave 0): the Gram tiles summed over the four blocks (the
//            transposes the inverse needs read transposed from LDS), the
//            blockwise 32 x 32 inverse, T diag(beta) into LDS, the M record;
//   phase 3 (each wave): its two W tiles, W = (T diag(beta))^T Khat.
// The phases are ordered by counters in the team's LDS (no workgroup
// barrier: the waves of other roles in the workgroup do not take part).
#pragma once

#include "kda_c32_dev.h"

namespace kda {

struct TeamLds {
    float part[4][6][256];       // [kb][tile][16 x 16 row-major]: A00, A11, A10, Q00t, Q11t, Q10t
    u32x2_t tb[3][2][64];        // T diag(beta) blocks 00, 11, 10: [block][hi/lo][lane]
    float beta[C32];
    int p1, p2, p3;              // phase counters: waves done with phase 1 / 2 / 3
};

__device__ __forceinline__ int team_lds_load(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// one increment per wave (from its first lane)
__device__ __forceinline__ void team_lds_inc(int *p) {
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(p, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Waits until *p >= want; false if the wait ran out (about a second).
__device__ __forceinline__ bool team_wait(const int *p, int want) {
    for (uint32_t n = 0; n < (1u << 23); ++n) {
        if (team_lds_load(p) >= want) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

__device__ __forceinline__ void team_init(TeamLds &T) {
    if ((threadIdx.x & 63) == 0) { T.p1 = 0; T.p2 = 0; T.p3 = 0; }
}

// One chunk (len tokens at token row t0) of head hh by the calling wave,
// channel block kb of the team; n: the team's count of chunks done before
// this one (the phase counters' targets).  dt_bias: per (head, channel),
// or [H] in the SG form.  Returns false if one of the waits ran out.
template <bool SG, bool NT>
__device__ __forceinline__ bool team_chunk(TeamLds &T, int kb, int n, const uint16_t *__restrict__ q,
                           const uint16_t *__restrict__ k, const uint16_t *__restrict__ g,
                           const uint16_t *__restrict__ beta, const float *__restrict__ dt_bias,
                           float A, float lb2, int64_t t0, int len, int H, int hh, int K,
                           uint8_t *__restrict__ rec) {
    typedef Rec32 R;
    const int l = threadIdx.x & 63;
    const int tok = l & 15, grp = l >> 4, cg = tok;
    bool ok = true;
    bool live[2];
    live[0] = tok < len;
    live[1] = 16 + tok < len;
    auto st16 = [&](const u32x4_t &v, int off) {
        if (NT) __builtin_nontemporal_store(v, (u32x4_t *)(rec + off));
        else *(u32x4_t *)(rec + off) = v;
    };
    u32x2_t eye;
    {
        const uint32_t one = 0x3f80u;
        const int d = tok - 4 * grp;
        eye[0] = (d == 0 ? one : 0u) | (d == 1 ? one << 16 : 0u);
        eye[1] = (d == 2 ? one : 0u) | (d == 3 ? one << 16 : 0u);
    }
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

    // ---- phase 1: this wave's channel block ----------------------------------
    Intra32Src in;
    intra32_src<SG>(in, q, k, g, beta, t0, len, H, hh, K);
    Intra32Blk cur;
    intra32_read<SG>(cur, in, kb);
    if (kb == 0) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const float x = bf16f((uint16_t)in.beta[b]);
            const float bv = __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * LOG2E));
            if (grp == 0) T.beta[16 * b + tok] = live[b] ? bv : 0.f;
        }
    }
    // dt_bias of this lane's eight channels in log2 units (zeros past K)
    float dtb2[8];
    if (SG) {
        const float d = dt_bias ? dt_bias[hh] * LOG2E : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) dtb2[i] = d;
    } else {
        const int c0 = 32 * kb + 8 * grp;
#pragma unroll
        for (int i = 0; i < 8; ++i) dtb2[i] = (dt_bias && c0 + i < K) ? dt_bias[(size_t)hh * K + c0 + i] * LOG2E : 0.f;
    }
    float gl[2][8];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        if (A > 0.f) {
            if (SG) {
                const float x2 = bf16f((uint16_t)in.gs[b]) * LOG2E + dtb2[0];
                const float u = fast_log2(1.f + fast_exp2(x2));
                const float la = fmaxf(-A * u, lb2);
                float s = live[b] ? la : 0.f;
                s += row_shr<1>(s);
                s += row_shr<2>(s);
                s += row_shr<4>(s);
                s += row_shr<8>(s);
#pragma unroll
                for (int i = 0; i < 8; ++i) gl[b][i] = s;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float x2 = elem(cur.g[b], i) * LOG2E + dtb2[i];
                    const float u = fast_log2(1.f + fast_exp2(x2));
                    const float la = fmaxf(-A * u, lb2);
                    gl[b][i] = live[b] ? la : 0.f;
                }
                row_prefix8(gl[b]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) gl[b][i] = 0.f;
        }
    }
    float F0[8], eg0[8], eg1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        F0[i] = fast_exp2(gl[0][i]);
        eg0[i] = row_last(F0[i]);
    }
    f32x4_t A00 = zero, A11 = zero, A10 = zero, Q00t = zero, Q11t = zero, Q10t = zero;
    u32x2_t kh[2][2];                  // Khat tiles t = 2kb + h of sub-block b (B layout, bf16)
    u32x4_t kf1, qfh1, qfl1;
    {
        u32x4_t kbh1, kbl1, kt1, qt1, kht1;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            float kF[2], qF[2], kB[2], kt[2], qt[2], khv[2];
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
                kt[e] = kF[e] * eg0[i];
                qt[e] = qF[e] * eg0[i];
                khv[e] = kv * (Bv * eg1[i]);
            }
            uint32_t h, lo;
            kf1[wd] = pack2(kF[0], kF[1]);
            split2(kB[0], kB[1], h, lo); kbh1[wd] = h; kbl1[wd] = lo;
            split2(qF[0], qF[1], h, lo); qfh1[wd] = h; qfl1[wd] = lo;
            kht1[wd] = pack2(khv[0], khv[1]);
            kt1[wd] = pack2(kt[0], kt[1]);
            qt1[wd] = pack2(qt[0], qt[1]);
        }
        st16(kt1, R::KT + ((kb * 2 + 1) * 64 + l) * 16);
        st16(qt1, R::QT + ((kb * 2 + 1) * 64 + l) * 16);
        A11 = mfma_k32(kf1, kbh1, A11);
        Q11t = mfma_k32(kbh1, qfh1, Q11t);
        Q11t = mfma_k32(kbh1, qfl1, Q11t);
        Q11t = mfma_k32(kbl1, qfh1, Q11t);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x2_t a = {kht1[2 * h], kht1[2 * h + 1]};
            const f32x4_t d = mfma_k16(a, eye, zero);
            kh[1][h] = {pack2(d[0], d[1]), pack2(d[2], d[3])};
        }
    }
    {
        u32x4_t kf0, kbh0, kbl0, qfh0, qfl0, ke0h, ke0l, kht0;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            float kF[2], qF[2], kB[2], ke[2], khv[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * wd + e;
                const float Bv = fast_exp2(-gl[0][i]);
                const float kv = elem(cur.k[0], i), qv = elem(cur.q[0], i);
                kF[e] = kv * F0[i];
                qF[e] = qv * F0[i];
                kB[e] = kv * Bv;
                ke[e] = kv * (Bv * eg0[i]);
                khv[e] = ke[e] * eg1[i];
            }
            uint32_t h, lo;
            kf0[wd] = pack2(kF[0], kF[1]);
            split2(kB[0], kB[1], h, lo); kbh0[wd] = h; kbl0[wd] = lo;
            split2(qF[0], qF[1], h, lo); qfh0[wd] = h; qfl0[wd] = lo;
            split2(ke[0], ke[1], h, lo); ke0h[wd] = h; ke0l[wd] = lo;
            kht0[wd] = pack2(khv[0], khv[1]);
        }
        st16(kf0, R::KT + ((kb * 2 + 0) * 64 + l) * 16);
        st16(qfh0, R::QT + ((kb * 2 + 0) * 64 + l) * 16);
        A00 = mfma_k32(kf0, kbh0, A00);
        A10 = mfma_k32(kf1, ke0h, A10);
        Q00t = mfma_k32(kbh0, qfh0, Q00t);
        Q00t = mfma_k32(kbh0, qfl0, Q00t);
        Q00t = mfma_k32(kbl0, qfh0, Q00t);
        Q10t = mfma_k32(ke0h, qfh1, Q10t);
        Q10t = mfma_k32(ke0h, qfl1, Q10t);
        Q10t = mfma_k32(ke0l, qfh1, Q10t);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x2_t a = {kht0[2 * h], kht0[2 * h + 1]};
            const f32x4_t d = mfma_k16(a, eye, zero);
            kh[0][h] = {pack2(d[0], d[1]), pack2(d[2], d[3])};
        }
    }
    // chunk decay 2^{Gam_0 + Gam_1} of this lane's channels (token-15 lanes)
    if (tok == 15) {
        f32x4_t g0, g1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            g0[i] = eg0[i] * eg1[i];
            g1[i] = eg0[4 + i] * eg1[4 + i];
        }
        const int ch = 32 * kb + 8 * grp;
        if (NT) {
            __builtin_nontemporal_store(g0, (f32x4_t *)(rec + R::GAM + ch * 4));
            __builtin_nontemporal_store(g1, (f32x4_t *)(rec + R::GAM + ch * 4 + 16));
        } else {
            *(f32x4_t *)(rec + R::GAM + ch * 4) = g0;
            *(f32x4_t *)(rec + R::GAM + ch * 4 + 16) = g1;
        }
    }
    // partial Gram tiles, row-major: lane l holds rows 4grp + j, column l%16
    {
        const f32x4_t tiles[6] = {A00, A11, A10, Q00t, Q11t, Q10t};
#pragma unroll
        for (int t = 0; t < 6; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) T.part[kb][t][(4 * grp + j) * 16 + cg] = tiles[t][j];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    team_lds_inc(&T.p1);

    // ---- phase 2: wave 0 -------------------------------------------------------
    if (kb == 0) {
        ok = ok && team_wait(&T.p1, 4 * (n + 1));
        // T.tb is rewritten below: every wave has read the previous chunk's
        ok = ok && team_wait(&T.p3, 4 * n);
        // sums over the four channel blocks; t: tile, tr: read transposed
        auto sum = [&](int t, bool tr) {
            f32x4_t s = zero;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    s[j] += tr ? T.part[b][t][cg * 16 + 4 * grp + j] : T.part[b][t][(4 * grp + j) * 16 + cg];
            return s;
        };
        const f32x4_t a00 = sum(0, false), a00t = sum(0, true);
        const f32x4_t a11 = sum(1, false), a11t = sum(1, true);
        const f32x4_t a10 = sum(2, false);
        const f32x4_t q00t = sum(3, false), q11t = sum(4, false), q10t = sum(5, false);
        float br[2][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) { br[0][j] = T.beta[4 * grp + j]; br[1][j] = T.beta[16 + 4 * grp + j]; }
        const float bc0 = T.beta[cg], bc1 = T.beta[16 + cg];
        f32x4_t I4, n0, n0t, n1, n1t, l10;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * grp + j;
            n0[j] = (cg < r) ? -br[0][j] * a00[j] : 0.f;
            n0t[j] = (r < cg) ? -bc0 * a00t[j] : 0.f;
            n1[j] = (cg < r) ? -br[1][j] * a11[j] : 0.f;
            n1t[j] = (r < cg) ? -bc1 * a11t[j] : 0.f;
            l10[j] = br[1][j] * a10[j];
            I4[j] = (r == cg) ? 1.f : 0.f;
        }
        f32x4_t T00, T00t, T11, T11t;
        neumann16(n0, n0t, I4, T00, T00t);
        neumann16(n1, n1t, I4, T11, T11t);
        const f32x4_t Ut = mm16(l10, T11t);            // (T11 L10)^T
        const f32x4_t T10 = -mm16(Ut, T00);            // -T11 L10 T00
        u32x2_t tb00h, tb00l, tb11h, tb11l, tb10h, tb10l;
        split2v(T00, bc0, tb00h, tb00l);
        split2v(T11, bc1, tb11h, tb11l);
        split2v(T10, bc0, tb10h, tb10l);
        T.tb[0][0][l] = tb00h; T.tb[0][1][l] = tb00l;
        T.tb[1][0][l] = tb11h; T.tb[1][1][l] = tb11l;
        T.tb[2][0][l] = tb10h; T.tb[2][1][l] = tb10l;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        team_lds_inc(&T.p2);
        // M = Aqk T diag(beta), as M^T blocks
        f32x4_t m00, m11;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m00[j] = (4 * grp + j <= cg) ? q00t[j] : 0.f;
            m11[j] = (4 * grp + j <= cg) ? q11t[j] : 0.f;
        }
        u32x2_t q00h, q00l, q11h, q11l, q10h, q10l;
        split2v(m00, 1.f, q00h, q00l);
        split2v(m11, 1.f, q11h, q11l);
        split2v(q10t, 1.f, q10h, q10l);
        const f32x4_t M00t = mfma3_k16(tb00h, tb00l, q00h, q00l, zero);
        const f32x4_t M11t = mfma3_k16(tb11h, tb11l, q11h, q11l, zero);
        f32x4_t M10t = mfma3_k16(tb00h, tb00l, q10h, q10l, zero);
        M10t = mfma3_k16(tb10h, tb10l, q11h, q11l, M10t);
        const u32x4_t m0 = {pack2(M00t[0], M00t[1]), pack2(M00t[2], M00t[3]), 0u, 0u};
        const u32x4_t m1 = {pack2(M10t[0], M10t[1]), pack2(M10t[2], M10t[3]),
                            pack2(M11t[0], M11t[1]), pack2(M11t[2], M11t[3])};
        st16(m0, R::M + l * 16);
        st16(m1, R::M + (64 + l) * 16);
    }

    // ---- phase 3: this wave's W tiles t = 2kb, 2kb + 1 ------------------------
    ok = ok && team_wait(&T.p2, n + 1);
    {
        const u32x2_t t00h = T.tb[0][0][l], t00l = T.tb[0][1][l];
        const u32x2_t t11h = T.tb[1][0][l], t11l = T.tb[1][1][l];
        const u32x2_t t10h = T.tb[2][0][l], t10l = T.tb[2][1][l];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4_t w0 = mfma_k16(t00h, kh[0][h], zero);
            w0 = mfma_k16(t00l, kh[0][h], w0);
            w0 = mfma_k16(t10h, kh[1][h], w0);
            w0 = mfma_k16(t10l, kh[1][h], w0);
            f32x4_t w1 = mfma_k16(t11h, kh[1][h], zero);
            w1 = mfma_k16(t11l, kh[1][h], w1);
            const u32x4_t o = {pack2(w0[0], w0[1]), pack2(w0[2], w0[3]), pack2(w1[0], w1[1]),
                               pack2(w1[2], w1[3])};
            st16(o, R::WT + ((2 * kb + h) * 64 + l) * 16);
        }
    }
    // every store of this wave acknowledged (and its LDS reads of T.tb done)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    team_lds_inc(&T.p3);
    return ok;
}

}  // namespace kda
