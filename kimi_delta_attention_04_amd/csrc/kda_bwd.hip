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
//   prep    (chunk slot, head), one wave  the chunk factors into the states
//           scan's record (Kt and Wm with the chunk decay, bf16) and
//           the reverse scan's bf16 record (Wm, scale Qt, -Kt, scale M^T),
//           in MFMA operand layouts
//   states  (sequence, head, column part)  forward scan on the forward
//           scan's structure (kda_bwd_scan.hip), storing the start state S0
//           of the even chunks of each sequence (bf16 rows) and every X (bf16)
//   rscan   (sequence, head, column part)  reverse scan of dS on the same
//           structure, beside the states scan on a second stream, storing
//           dS1 of the odd chunks and of the last one (bf16 rows), writing
//           dv (= dX, which the chunk kernel reads back) and the
//           initial-state gradient
//   chunk   (chunk slot, head), one wave  the products with S0 / dS1 and the
//           in-chunk backward on bf16 MFMAs with (hi, lo) operands: dq, dk,
//           dg, dbeta, per-chunk dA_log / ddt_bias sums
//   reduce  (head)  sums the per-chunk parameter gradients in slot order
// Every sum runs in a fixed order, so results are bitwise reproducible.
#include <math.h>

#include <mutex>

#include "kda_device.h"
#include "kda_bwd_dev.h"
#include "kda_intra_dev.h"                            // intra_load, mm16, the decay prefix
#include "kda_launch.h"

namespace kda {

namespace {

constexpr float LN2 = 0.6931471805599453f;

// Token range of chunk slot `slot`: returns its token count (0 for a gap
// slot) and the first token row in t0; also the chunk's index within its
// sequence (ci) and the sequence's end row.
__device__ int slot_chunk(const int32_t *cu, int N, int T, int64_t slot, int64_t &t0, int &ci,
                          int64_t &end) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seq_slot0(cu, mid, T) <= slot) lo = mid; else hi = mid - 1;
    }
    int64_t start;
    seq_range(cu, lo, T, start, end);
    ci = (int)(slot - seq_slot0(cu, lo, T));
    t0 = start + (int64_t)ci * CS;
    return t0 >= end ? 0 : (int)min((int64_t)CS, end - t0);
}
__device__ int slot_chunk(const int32_t *cu, int N, int T, int64_t slot, int64_t &t0) {
    int ci;
    int64_t end;
    return slot_chunk(cu, N, T, slot, t0, ci, end);
}

// ---------------------------------------------------------------------------
// chunk: one wave per (chunk slot, head), everything that needs S0 and dS1
// of the chunk, then the in-chunk backward down to the inputs.  No barrier:
// the wave keeps its operands in MFMA register layouts and moves 16 x 16
// tiles between layouts through a few hundred bytes of its own LDS.
//
// Layouts (lane l, tok = l%16, grp = l/16):
//   token-per-lane  lane l holds token tok, channels 32kb + 8grp + i
//                   (i = 0..7) of each 32-channel block kb: the A and B
//                   operand layout of a 16x16x32 MFMA contracting over
//                   channels (or value columns), as in the intra stage
//   tile            16 x 16 matrices in accumulator layout: rows 4grp + j,
//                   column tok
//   W^T             tile t of a tokens x channels matrix: tokens 4grp + j,
//                   channel chan(t, tok) (kda_device.h), the A operand
//                   layout of a 16x16x16 MFMA contracting over tokens
// A product whose rows are the state rows chan(t, .) of tiles 2kb and
// 2kb + 1 lands, in accumulator layout, in the token-per-lane layout of
// block kb; an identity MFMA turns token-per-lane bf16 into W^T bf16 and
// back, exactly.  fp32 operands enter the bf16 MFMAs as (hi, lo) pairs with
// three products (hi hi + hi lo + lo hi), about 16 significant bits.
// ---------------------------------------------------------------------------
// Per key channel of head dimension KD.  20160 bytes at KD = 128, so that
// eight one-wave workgroups (two per SIMD, as the registers allow) fit a
// compute unit's 160 KB in 512-byte allocation units.
template <int KD>
struct ChunkWaveLds {
    float beta[CS];
    float daq[CS];                    // diagonal of dAqk
    float dtb[KD];                    // dt_bias in log2 units
    union {                           // (one wave: program order separates the two)
        float gnb[KD];                // the state products: chunk decay of the
                                      // neighbour chunk whose state is used
        float gam[KD];                // from the chunk factors on: e^{G_last} per key channel
    };
    float gl[KD];                     // G_last in log2 units
    float dgs[KD];                    // diag(dS1 S0^T) per key channel, in two parts
    float dgs2[KD];
    float tile[CS][CS + 1];           // 16 x 16 transposes
    f32x4_t qs[KD / 16][64];          // (dO S0^T)^T and (dX S0^T)^T per state row
    f32x4_t ks[KD / 16][64];          // tile and lane, between their two phases
};

// The tile layout of Z -> the tile layout of Z^T, through the wave's LDS.
__device__ __forceinline__ f32x4_t tr16(float (&b)[CS][CS + 1], f32x4_t x) {
    const int l = threadIdx.x & 63, tok = l & 15, grp = l >> 4;
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 4; ++j) b[4 * grp + j][tok] = x[j];
    wave_lds_sync();
    f32x4_t y;
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = b[tok][4 * grp + j];
    return y;
}

// (hi, lo) bf16 parts of a tile (four fp32) and of eight fp32 values.
__device__ __forceinline__ void split4(f32x4_t x, u32x2_t &hi, u32x2_t &lo) {
    uint32_t h0, l0, h1, l1;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    hi = {h0, h1};
    lo = {l0, l1};
}
__device__ __forceinline__ void split8(f32x4_t a, f32x4_t b, u32x4_t &hi, u32x4_t &lo) {
    uint32_t h, w;
    split2(a[0], a[1], h, w); hi[0] = h; lo[0] = w;
    split2(a[2], a[3], h, w); hi[1] = h; lo[1] = w;
    split2(b[0], b[1], h, w); hi[2] = h; lo[2] = w;
    split2(b[2], b[3], h, w); hi[3] = h; lo[3] = w;
}
// C + A B from (hi, lo) parts: hi hi + hi lo + lo hi.
__device__ __forceinline__ f32x4_t mm3_k16(u32x2_t ah, u32x2_t al, u32x2_t bh, u32x2_t bl, f32x4_t c) {
    c = mfma_k16(ah, bh, c);
    c = mfma_k16(ah, bl, c);
    return mfma_k16(al, bh, c);
}
__device__ __forceinline__ f32x4_t mm3_k32(u32x4_t ah, u32x4_t al, u32x4_t bh, u32x4_t bl, f32x4_t c) {
    c = mfma_k32(ah, bh, c);
    c = mfma_k32(ah, bl, c);
    return mfma_k32(al, bh, c);
}

// Sum over the 16 lanes of each DPP row, in every lane of the row.
template <int SH>
__device__ __forceinline__ float row_ror(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x120 + SH, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum16(float x) {
    x += row_ror<8>(x);
    x += row_ror<4>(x);
    x += row_ror<2>(x);
    return x + row_ror<1>(x);
}
// Inclusive suffix sum over the 16 lanes of each DPP row (lane i: lanes i..15).
template <int SH>
__device__ __forceinline__ float row_shl(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x100 + SH, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_suffix16(float x) {
    x += row_shl<1>(x);
    x += row_shl<2>(x);
    x += row_shl<4>(x);
    return x + row_shl<8>(x);
}

// The identity as a 16x16x16 B operand: mfma_k16(a, eye) is the tile layout
// of the matrix whose A operand is a.
__device__ __forceinline__ u32x2_t identity_b() {
    const int l = threadIdx.x & 63;
    const int d = (l & 15) - 4 * (l >> 4);
    const uint32_t one = 0x3f80u;                           // bf16 1.0
    u32x2_t e;
    e[0] = (d == 0 ? one : 0u) | (d == 1 ? one << 16 : 0u);
    e[1] = (d == 2 ? one : 0u) | (d == 3 ? one << 16 : 0u);
    return e;
}

// Four bf16 channels 32kb + 8grp + 4hh + j (j = 0..3) of this lane's token
// (the A operand layout of a 16x16x16 MFMA) -> the W^T layout of tile
// 2kb + hh, exactly.
__device__ __forceinline__ u32x2_t to_wt(u32x2_t a, u32x2_t eye) {
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    const f32x4_t d = mfma_k16(a, eye, z);
    return {pack2(d[0], d[1]), pack2(d[2], d[3])};
}

// Log-decay in log2 units, as the forward's intra stage forms it, of the NI
// channels 32kb + 8grp + i0 + i of this lane's token: per (token, channel)
// x2 = (g + dt_bias) log2 e, the clamped gate max(-A log2(1 + 2^x2),
// lb log2 e) (zero on padding rows), and its inclusive cumulative sum G over
// the chunk's tokens (across the 16 lanes of the DPP row).  U, SG (when
// given): the gate before its clamp, y = -A u with u = log2(1 + 2^x2), as u,
// and sigmoid(g + dt_bias) = 2^(x2 - u) (since 2^u = 1 + 2^x2).
template <int NI>
__device__ __forceinline__ void block_decay(const u32x4_t gw, const float *__restrict__ dtb_lds,
                                            int kb, int i0, float A, float lb2, bool live,
                                            float (&G)[NI], float *U = nullptr, float *SG = nullptr) {
    const int grp = (threadIdx.x & 63) >> 4;
    if (A > 0.f) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const float x2 = elem(gw, i0 + i) * LOG2E + dtb_lds[32 * kb + 8 * grp + i0 + i];
            const float u = fast_log2(1.f + fast_exp2(x2));
            const float la = fmaxf(-A * u, lb2);
            G[i] = live ? la : 0.f;
            if (U) U[i] = u;
            if (SG) SG[i] = fast_exp2(x2 - u);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) G[i] += row_shr<1>(G[i]);
#pragma unroll
        for (int i = 0; i < NI; ++i) G[i] += row_shr<2>(G[i]);
#pragma unroll
        for (int i = 0; i < NI; ++i) G[i] += row_shr<4>(G[i]);
#pragma unroll
        for (int i = 0; i < NI; ++i) G[i] += row_shr<8>(G[i]);
    } else {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            G[i] = 0.f;
            if (U) U[i] = 0.f;
            if (SG) SG[i] = 0.f;
        }
    }
}

// SCALAR: the Gated DeltaNet form (one gate value per token and head, g and
// dt_bias broadcast over the channels by the caller): the gate gradient is
// summed over the channels in fp32 and written to dgs [token, head] in bf16,
// and the channel-wise dg is not written.
template <int KD, bool SCALAR = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(KD > 128 ? 1 : 2))) void bwd_chunk_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ g, const uint16_t *__restrict__ beta,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float lb, float scale,
    const uint16_t *__restrict__ dout, const int32_t *__restrict__ cu, int N, int T, int H,
    const uint16_t *__restrict__ st0, const uint16_t *__restrict__ dst1,
    const uint16_t *__restrict__ xws, const uint16_t *__restrict__ dvv,
    const uint8_t *__restrict__ srec, const uint8_t *__restrict__ rrec,
    uint16_t *__restrict__ dq, uint16_t *__restrict__ dk, uint16_t *__restrict__ dg,
    uint16_t *__restrict__ dbeta, float *__restrict__ part_alog, float *__restrict__ part_dtb,
    uint16_t *__restrict__ dgs)
{
    constexpr int NKB = KD / 32;                            // channel blocks = 32-column steps
    constexpr int NT = 2 * NKB;                             // state row tiles
    constexpr int PD = bwd_pd_stride<KD>();                 // dt_bias partial sums per (slot, head)
    __shared__ __attribute__((aligned(16))) ChunkWaveLds<KD> L;
    const int64_t slot = blockIdx.x / (unsigned)H;
    const int h = (int)(blockIdx.x % (unsigned)H);
    const int l = threadIdx.x, tok = l & 15, grp = l >> 4;
    const size_t sh = (size_t)slot * H + h;
    int64_t t0, tend;
    int ci;
    const int len = slot_chunk(cu, N, T, slot, t0, ci, tend);
    if (len == 0) {                                         // gap slot: zero partial sums
#pragma unroll
        for (int i = 0; i < PD; i += 64) part_dtb[sh * PD + i + l] = 0.f;
        if (l == 0) part_alog[sh] = 0.f;
        return;
    }
    const bool live = tok < len;
    const float A = expf(A_log[h]);
    const float lb2 = lb * LOG2E;
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    const u32x2_t eye = identity_b();

    // token rows of this chunk ([token, head, channel] tensors): loads past
    // the chunk's tokens return zeros, stores there are dropped
    const size_t rowe = (size_t)H * KD;
    const uint32_t rbytes = (uint32_t)(((size_t)(len - 1) * rowe + KD) * 2);
    const size_t rbase = ((size_t)t0 * H + h) * KD;
    const __amdgpu_buffer_rsrc_t r_do = make_rsrc(dout + rbase, rbytes);
    auto row_off = [&](int kb) { return (int)((tok * rowe + 32 * kb + 8 * grp) * 2); };

    // ---- products with the states ------------------------------------------
    // The states scan stores S0 of a sequence's even chunks (index within the
    // sequence) and the reverse scan dS1 of its odd chunks and of its last
    // one.  An odd chunk takes S0 of the chunk before (p) and an even chunk
    // other than the last takes dS1 of the chunk after (n), through the
    // chunk steps
    //   S0  = Gam_p S0_p + Wm_p^T X_p,
    //   dS1 = Gam_n dS1_n + scale Qt_n^T dO_n - Kt_n^T dX_n,
    // so each product with the state it lacks is the same product with the
    // stored one, scaled per channel, plus 16 x 16 by 16 x 128 terms from the
    // neighbour's X, dO, dX and its records (Wm_p, the chunk decays, scale
    // Qt_n and -Kt_n).  Neighbouring chunks of a head are 8 H workgroups
    // apart, so their reads of the shared state rows meet in one L2.
    //
    // Over the value columns in 32-column steps s, per state row tile t:
    //   (dO S0^T)^T, (dX S0^T)^T   rows chan(t, .): token-per-lane results
    //   dWm = X dS1^T              W^T layout (A = X, B = dS1 rows)
    //   diag(dS1 S0^T)             the diagonal of S0 rows x dS1 rows^T
    // and once: dM / scale = dO X^T (tile).  The stored states are bf16 rows
    // [16-column part][KD rows][16]; the A operand of tile t, step s is row
    // chan(t, tok), columns 32s + 8grp .. +7.
    const bool odd = (ci & 1) != 0;                         // S0 from the chunk before
    const bool reb = !odd && t0 + CS < tend;                // dS1 from the chunk after
    typedef RecLayout<KD> R;
    typedef StatesRecT<KD> SR;
    const size_t shS = odd ? sh - H : sh, shD = reb ? sh + H : sh;
    // the neighbour's chunk decay (p's for an odd chunk, n's for a rebuilt dS1)
    {
        const uint8_t *gsrc = srec + (odd ? shS : shD) * SR::BYTES + SR::GAM;
#pragma unroll
        for (int c = 2 * l; c < KD; c += 128) *(u32x2_t *)&L.gnb[c] = *(const u32x2_t *)(gsrc + 4 * c);
    }
    f32x4_t dM = zero;
    u32x2_t wwh[NT], wwl[NT];
    {
        const uint16_t *S0 = st0 + shS * KD * KD + (size_t)(l >> 5) * KD * 16 + 8 * ((l >> 4) & 1);
        const uint16_t *DS = dst1 + shD * KD * KD + (size_t)(l >> 5) * KD * 16 + 8 * ((l >> 4) & 1);
        auto sld = [&](const uint16_t *b, int s, int t) {
            return *(const u32x4_t *)&b[((size_t)2 * s * KD + state_chan(t, tok)) * 16];
        };
        // the token-per-lane operands of every step: this chunk's dO, X, dX;
        // e1, e2: the neighbour's X (odd) or dO, dX (rebuilt dS1)
        const int len_n = reb ? (int)min((int64_t)CS, tend - t0 - CS) : 1;
        const size_t rbase_n = rbase + (size_t)CS * rowe;
        const uint32_t rbytes_n = (uint32_t)(((size_t)(len_n - 1) * rowe + KD) * 2);
        const __amdgpu_buffer_rsrc_t r_dx = make_rsrc(dvv + rbase, rbytes);
        const __amdgpu_buffer_rsrc_t r_don = make_rsrc(dout + rbase_n, reb ? rbytes_n : 0u);
        const __amdgpu_buffer_rsrc_t r_dxn = make_rsrc(dvv + rbase_n, reb ? rbytes_n : 0u);
        const uint16_t *xr = xws + sh * CS * KD + tok * KD + 8 * grp;
        const uint16_t *xp = xws + shS * CS * KD + tok * KD + 8 * grp;
        u32x4_t ob[NKB], xb[NKB], db[NKB], e1[NKB], e2[NKB];
#pragma unroll
        for (int st = 0; st < NKB; ++st) {
            ob[st] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r_do, row_off(st), 0, 0));
            xb[st] = *(const u32x4_t *)&xr[32 * st];
            db[st] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r_dx, row_off(st), 0, 0));
            if (odd) {
                e1[st] = *(const u32x4_t *)&xp[32 * st];
                e2[st] = e1[st];
            } else {
                e1[st] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r_don, row_off(st), 0, 0));
                e2[st] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r_dxn, row_off(st), 0, 0));
            }
        }
        // 16 x 16 products over the value columns: dM; for an odd chunk
        // Z1 = X_p dO^T and Z2 = X_p dX^T (tiles); for a rebuilt dS1
        // Z1 = dO_n X^T and Z2 = dX_n X^T (tiles, i.e. X dO_n^T and X dX_n^T in
        // the A operand layout)
        f32x4_t Z1 = zero, Z2 = zero;
#pragma unroll
        for (int st = 0; st < NKB; ++st) {
            dM = mfma_k32(ob[st], xb[st], dM);
            if (odd) {
                Z1 = mfma_k32(e1[st], ob[st], Z1);
                Z2 = mfma_k32(e1[st], db[st], Z2);
            } else if (reb) {
                Z1 = mfma_k32(e1[st], xb[st], Z1);
                Z2 = mfma_k32(e2[st], xb[st], Z2);
            }
        }
        u32x2_t z1h, z1l, z2h, z2l;
        split4(Z1, z1h, z1l);
        split4(Z2, z2h, z2l);
        wave_lds_sync();                                    // the neighbour's decay staged
        u32x4_t sa[NKB], sd[NKB];
#pragma unroll
        for (int st = 0; st < NKB; ++st) { sa[st] = sld(S0, st, 0); sd[st] = sld(DS, st, 0); }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            u32x4_t na[NKB], nd[NKB];                       // the next tile's rows in flight
            if (t + 1 < NT) {
#pragma unroll
                for (int st = 0; st < NKB; ++st) { na[st] = sld(S0, st, t + 1); nd[st] = sld(DS, st, t + 1); }
            }
            f32x4_t Qa = zero, Ka = zero, Wa = zero, Ea = zero, Eb = zero, Dg = zero;
#pragma unroll
            for (int st = 0; st < NKB; ++st) {
                Qa = mfma_k32(sa[st], ob[st], Qa);
                Ka = mfma_k32(sa[st], db[st], Ka);
                Wa = mfma_k32(xb[st], sd[st], Wa);
                if (odd) {
                    Ea = mfma_k32(e1[st], sd[st], Ea);          // X_p dS1^T (W^T layout)
                } else if (reb) {
                    Ea = mfma_k32(sa[st], e1[st], Ea);          // (dO_n S0^T)^T
                    Eb = mfma_k32(sa[st], e2[st], Eb);          // (dX_n S0^T)^T
                }
                // S0 rows against dS1 rows (the same registers are the B
                // operand of their transpose): diag(dS1 S0^T) on the diagonal
                Dg = mfma_k32(sa[st], sd[st], Dg);
            }
            // lane (tok, grp = tok / 4) holds the diagonal element of channel
            // chan(t, tok) in slot tok % 4; summed over the lane groups
            float dg = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) dg = 4 * grp + j == tok ? Dg[j] : dg;
            dg += __shfl_xor(dg, 16, 64);
            dg += __shfl_xor(dg, 32, 64);                   // channel chan(t, tok)
            const int ct = state_chan(t, tok);
            float dg2[4] = {0.f, 0.f, 0.f, 0.f};            // channels chan(t, 4grp + j)
            if (odd) {
                // S0 = Gam_p S0_p + Wm_p^T X_p: rows chan(t, 4grp + j) of the
                // products scale by their decay, plus Wm_p^T (X_p dO^T); the
                // decay's own term adds X_p dS1^T o Wm_p summed over tokens
                const u32x2_t wmp = *(const u32x2_t *)(srec + shS * SR::BYTES + SR::WTH +
                                                       ((t >> 1) * 64 + l) * 16 + 8 * (t & 1));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float gr = L.gnb[state_chan(t, 4 * grp + j)];
                    Qa[j] *= gr;
                    Ka[j] *= gr;
                }
                Qa = mfma_k16(wmp, z1h, Qa);
                Qa = mfma_k16(wmp, z1l, Qa);
                Ka = mfma_k16(wmp, z2h, Ka);
                Ka = mfma_k16(wmp, z2l, Ka);
                float wx = Ea[0] * bf16lo(wmp[0]) + Ea[1] * bf16hi(wmp[0]) +
                           Ea[2] * bf16lo(wmp[1]) + Ea[3] * bf16hi(wmp[1]);
                wx += __shfl_xor(wx, 16, 64);
                wx += __shfl_xor(wx, 32, 64);
                dg = L.gnb[ct] * dg + wx;
            } else if (reb) {
                // dS1 = Gam_n dS1_n + scale Qt_n^T dO_n - Kt_n^T dX_n: dWm's
                // columns scale by their decay, plus (X dO_n^T) scale Qt_n and
                // (X dX_n^T) (-Kt_n); diag(dS1 S0^T) takes the decay and the
                // sums over tokens of scale Qt_n o (dO_n S0^T) and
                // -Kt_n o (dX_n S0^T)
                const size_t ro = shD * R::BYTES + ((t >> 1) * 64 + l) * 16 + 8 * (t & 1);
                const u32x2_t qtn = *(const u32x2_t *)(rrec + ro + R::QT);
                const u32x2_t ktn = *(const u32x2_t *)(rrec + ro + R::WT);
                const float gc = L.gnb[ct];
#pragma unroll
                for (int j = 0; j < 4; ++j) Wa[j] *= gc;
                Wa = mfma_k16(z1h, qtn, Wa);
                Wa = mfma_k16(z1l, qtn, Wa);
                Wa = mfma_k16(z2h, ktn, Wa);
                Wa = mfma_k16(z2l, ktn, Wa);
                const f32x4_t qtl = mfma_k16(qtn, eye, zero);   // token tok, channels chan(t, 4grp + j)
                const f32x4_t ktl = mfma_k16(ktn, eye, zero);
#pragma unroll
                for (int j = 0; j < 4; ++j) dg2[j] = row_sum16(Ea[j] * qtl[j] + Eb[j] * ktl[j]);
                dg = gc * dg;
            }
            if (grp == 0) L.dgs[ct] = dg;
            if (tok == 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) L.dgs2[state_chan(t, 4 * grp + j)] = dg2[j];
            }
            L.qs[t][l] = Qa;
            L.ks[t][l] = Ka;
            split4(Wa, wwh[t], wwl[t]);
            if (t + 1 < NT) {
#pragma unroll
                for (int st = 0; st < NKB; ++st) { sa[st] = na[st]; sd[st] = nd[st]; }
            }
        }
    }

    // ---- chunk factors, and Y = Kb Gam dWm^T --------------------------------
    stage_dtb<false, KD>(L.dtb, dt_bias, h, KD);
    IntraInT<NKB> in;
    intra_load<false, KD>(in, q, k, g, beta, t0, len, H, h, KD);
    {
        const float x = bf16f((uint16_t)in.beta);
        const float b = __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * LOG2E));
        if (grp == 0) L.beta[tok] = live ? b : 0.f;
    }
    wave_lds_sync();                                        // dt_bias staged
    f32x4_t Akk = zero, AkkT = zero, Aqk = zero, Y = zero;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        float G[8];
        block_decay<8>(in.g[kb], L.dtb, kb, 0, A, lb2, live, G);
        if (tok == CS - 1) {
            f32x4_t g0, g1, l0, l1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                g0[i] = fast_exp2(G[i]); g1[i] = fast_exp2(G[4 + i]);
                l0[i] = G[i]; l1[i] = G[4 + i];
            }
            *(f32x4_t *)&L.gam[32 * kb + 8 * grp] = g0;
            *(f32x4_t *)&L.gam[32 * kb + 8 * grp + 4] = g1;
            *(f32x4_t *)&L.gl[32 * kb + 8 * grp] = l0;
            *(f32x4_t *)&L.gl[32 * kb + 8 * grp + 4] = l1;
        }
        wave_lds_sync();
        float gl[8];
        *(f32x4_t *)&gl[0] = *(const f32x4_t *)&L.gl[32 * kb + 8 * grp];
        *(f32x4_t *)&gl[4] = *(const f32x4_t *)&L.gl[32 * kb + 8 * grp + 4];
        // The Grams are formed from Kt, Qt and Kb rescaled by e^{-G_last/2}
        // and e^{G_last/2} per channel, which leaves Kt Kb^T and Qt Kb^T
        // unchanged: at the lowest lower bound G_last reaches -86 (natural
        // log), where k e^G falls among the denormals and the bf16 (hi, lo)
        // parts of such a value keep only a few bits; rescaled, every factor
        // stays within e^{+-43}.  Kb Gam = k e^{G_last - G} needs no rescale.
        u32x4_t kth, ktl, qth, qtl, kbh, kbl, kgh, kgl;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            float kt[2], qt[2], kbv[2], kg[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * wd + e;
                const float gh = 0.5f * gl[i];
                const float eg = fast_exp2(G[i] - gh), egi = fast_exp2(gh - G[i]);
                const float kv = elem(in.k[kb], i), qv = elem(in.q[kb], i);
                kt[e] = kv * eg;
                qt[e] = qv * eg;
                kbv[e] = kv * egi;
                kg[e] = kv * fast_exp2(gl[i] - G[i]);
            }
            uint32_t a, b;
            split2(kt[0], kt[1], a, b); kth[wd] = a; ktl[wd] = b;
            split2(qt[0], qt[1], a, b); qth[wd] = a; qtl[wd] = b;
            split2(kbv[0], kbv[1], a, b); kbh[wd] = a; kbl[wd] = b;
            split2(kg[0], kg[1], a, b); kgh[wd] = a; kgl[wd] = b;
        }
        Akk = mm3_k32(kth, ktl, kbh, kbl, Akk);             // Akk[r][c]  = Kt_r . Kb_c
        AkkT = mm3_k32(kbh, kbl, kth, ktl, AkkT);           // AkkT[r][c] = Akk[c][r]
        Aqk = mm3_k32(qth, qtl, kbh, kbl, Aqk);             // Aqk[r][c]  = Qt_r . Kb_c
        // dWm of block kb token-per-lane, through the identity (exact)
        u32x4_t dwh, dwl;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const f32x4_t a = mfma_k16(wwh[2 * kb + hh], eye, zero), b = mfma_k16(wwl[2 * kb + hh], eye, zero);
            dwh[2 * hh] = pack2(a[0], a[1]);
            dwh[2 * hh + 1] = pack2(a[2], a[3]);
            dwl[2 * hh] = pack2(b[0], b[1]);
            dwl[2 * hh + 1] = pack2(b[2], b[3]);
        }
        Y = mm3_k32(kgh, kgl, dwh, dwl, Y);                 // (Kb Gam dWm^T)[r][c]
    }

    // ---- the 16 x 16 chain (tiles; row r = 4grp + j, column tok) ------------
    float br[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) br[j] = L.beta[4 * grp + j];
    const float bc = L.beta[tok];
    f32x4_t Tm;
    {
        // T = (I + diag(beta) strict_lower(Akk))^-1 = (I - N)^-1, N strictly
        // lower hence nilpotent: (I + N)(I + N^2)(I + N^4)(I + N^8)
        f32x4_t N1, N1t, I;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * grp + j;
            N1[j] = tok < r ? -br[j] * Akk[j] : 0.f;
            N1t[j] = r < tok ? -bc * AkkT[j] : 0.f;
            I[j] = r == tok ? 1.f : 0.f;
        }
        const f32x4_t N2 = mm16(N1t, N1), N2t = mm16(N1, N1t);
        const f32x4_t Q12t = mm16(I + N2, I + N1t);         // ((I+N)(I+N^2))^T
        const f32x4_t N4 = mm16(N2t, N2), N4t = mm16(N2, N2t);
        const f32x4_t Q3t = mm16(I + N4, Q12t);
        const f32x4_t N8 = mm16(N4t, N4);
        Tm = mm16(Q3t, I + N8);
    }
    const f32x4_t Tt = tr16(L.tile, Tm);                   // T^T
    f32x4_t Pt, Aq, Amt, dMs;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * grp + j;
        Pt[j] = Tt[j] * br[j];                              // P^T, P = T diag(beta)
        Aq[j] = tok <= r ? Aqk[j] : 0.f;                    // lower_incl(Qt Kb^T)
        Amt[j] = r < tok ? AkkT[j] : 0.f;                   // A^T, A = strict_lower(Kt Kb^T)
        dMs[j] = scale * dM[j];
    }
    // M = Aqk P:  dAqk = lower_incl(dM P^T),  dP = Aqk^T dM (+ Y from Wm = P^T Kb Gam)
    f32x4_t dAqk = mm16(tr16(L.tile, dMs), Pt);
    const f32x4_t dP = mm16(Aq, dMs) + Y;
    // The diagonal of Aqk, Qt_r . Kb_r = q_r . k_r, does not depend on the
    // decay: its terms in dG (through Qt and through Kb) cancel exactly.
    // Formed in the products they would cancel only to the products'
    // rounding, which under strong decay is larger than dG itself; so the
    // products take dAqk strictly lower and the diagonal's gradients enter
    // dq and dk directly (dAqk[r][r] k_r and dAqk[r][r] q_r).
    f32x4_t dT;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * grp + j;
        if (tok == r) L.daq[tok] = dAqk[j];
        dAqk[j] = tok < r ? dAqk[j] : 0.f;
        dT[j] = dP[j] * bc;                                 // P = T diag(beta)
    }
    // T = (I + L)^-1:  dL = -T^T (dT T^T), strictly lower;  L = diag(beta) A
    const f32x4_t Y2 = mm16(tr16(L.tile, dT), Tt);
    f32x4_t dL = mm16(Tm, Y2), dA;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        dL[j] = tok < 4 * grp + j ? -dL[j] : 0.f;
        dA[j] = br[j] * dL[j];
    }
    {
        // beta enters P (column sums of dP o T) and L (row sums of dL o A)
        const f32x4_t dLt = tr16(L.tile, dL);
        float db = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) db += dP[j] * Tm[j] + dLt[j] * Amt[j];
        db += __shfl_xor(db, 16, 64);
        db += __shfl_xor(db, 32, 64);
        if (grp == 0 && live) dbeta[(size_t)(t0 + tok) * H + h] = tobf16(db * bc * (1.f - bc));
    }
    // B operands of the per-channel products
    u32x2_t qAh, qAl, aAh, aAl, pTh, pTl, dQh, dQl, dAh, dAl;
    split4(tr16(L.tile, dAqk), qAh, qAl);                  // dAqk^T
    split4(tr16(L.tile, dA), aAh, aAl);                    // dA^T
    split4(Pt, pTh, pTl);
    split4(dAqk, dQh, dQl);
    split4(dA, dAh, dAl);

    // ---- per state row tile t (channels 32kb + 8grp + 4hh + j of each
    // token, kb = t/2, hh = t%2): gradients of Qt, Kt, Kb, then q, k, the gate
    const __amdgpu_buffer_rsrc_t r_dq = make_rsrc(dq + rbase, rbytes);
    const __amdgpu_buffer_rsrc_t r_dk = make_rsrc(dk + rbase, rbytes);
    const __amdgpu_buffer_rsrc_t r_dg = make_rsrc(dg + rbase, rbytes);
    float pa = 0.f;
    float gsum = 0.f;                                       // SCALAR: this lane's channels of dg
    u32x4_t oq, ok, og;                                     // one 16-byte row piece of each output
    u32x4_t gq, kq, qq;                                     // and of each input, block kb
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int kb = t >> 1, hh = t & 1, c0 = 32 * kb + 8 * grp + 4 * hh;
        if (hh == 0) { gq = in.g[kb]; kq = in.k[kb]; qq = in.q[kb]; }
        float G[4], U[4], SG[4];
        block_decay<4>(gq, L.dtb, kb, 4 * hh, A, lb2, live, G, U, SG);
        // as in the factors: Kt, Qt, Kb rescaled by e^{-+G_last/2} (rs, ri) for
        // the products with the 16 x 16 gradients, whose results are then
        // scaled back into dq = dQt e^G and dk = dKt e^G + dKb e^-G directly
        const f32x4_t glv = *(const f32x4_t *)&L.gl[c0];
        float e[4], rs[4], ri[4], kg[4], kv[4], qv[4], kt[4], qt[4], kbv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float gh = 0.5f * glv[j];
            e[j] = fast_exp2(G[j]);
            rs[j] = fast_exp2(G[j] - gh);
            ri[j] = fast_exp2(gh - G[j]);
            kg[j] = fast_exp2(glv[j] - G[j]);               // e^{G_last - G}
            kv[j] = elem(kq, 4 * hh + j);
            qv[j] = elem(qq, 4 * hh + j);
            kt[j] = kv[j] * rs[j];
            qt[j] = qv[j] * rs[j];
            kbv[j] = kv[j] * ri[j];
        }
        // (hi, lo) bf16 of the four channels: the A operand of the identity
        // that yields their W^T tile
        u32x2_t kth, ktl, qth, qtl, kbh, kbl;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            uint32_t a, b;
            split2(kt[2 * w], kt[2 * w + 1], a, b); kth[w] = a; ktl[w] = b;
            split2(qt[2 * w], qt[2 * w + 1], a, b); qth[w] = a; qtl[w] = b;
            split2(kbv[2 * w], kbv[2 * w + 1], a, b); kbh[w] = a; kbl[w] = b;
        }
        const u32x2_t bwh = to_wt(kbh, eye), bwl = to_wt(kbl, eye);
        const u32x2_t qwh = to_wt(qth, eye), qwl = to_wt(qtl, eye);
        const u32x2_t kwh = to_wt(kth, eye), kwl = to_wt(ktl, eye);
        // rows chan(t, .) of (dAqk Kb)^T, (dA Kb)^T, (P dWm)^T and
        // (dAqk^T Qt + dA^T Kt)^T: this lane's token, channels c0 + j
        const f32x4_t pq = mm3_k16(bwh, bwl, qAh, qAl, zero);
        const f32x4_t pk = mm3_k16(bwh, bwl, aAh, aAl, zero);
        const f32x4_t pg = mm3_k16(wwh[t], wwl[t], pTh, pTl, zero);
        const f32x4_t pb = mm3_k16(kwh, kwl, dAh, dAl, mm3_k16(qwh, qwl, dQh, dQl, zero));
        const f32x4_t qs = L.qs[t][l], ks = L.ks[t][l];
        const f32x4_t gm = *(const f32x4_t *)&L.gam[c0];
        const f32x4_t dgs = *(const f32x4_t *)&L.dgs[c0] + *(const f32x4_t *)&L.dgs2[c0];
        const float daq = L.daq[tok];
        float vq[4], vk[4], vg[4], pd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // dQt e^G, dKt e^G and dKb e^-G (dKb = dAqk^T Qt + dA^T Kt + Gam P dWm),
            // without the diagonal of dAqk
            const float dQe = scale * qs[j] * e[j] + pq[j] * rs[j];
            const float dKe = pk[j] * rs[j] - ks[j] * e[j];
            const float dKi = pb[j] * ri[j] + pg[j] * kg[j];
            // dG = dKt Kt + dQt Qt - dKb Kb, from the scaled terms
            const float dG = dQe * qv[j] + (dKe - dKi) * kv[j];
            // the chunk decay times its gradient: diag(dS1 S0^T) and the Wm
            // path's sum over tokens of (P dWm) o Kb Gam
            const float gdg = gm[j] * dgs[j] + row_sum16(pg[j] * kv[j] * kg[j]);
            // per-token log-decay (natural log): reverse cumulative sum of dG,
            // plus the chunk decay's term, which every token's decay enters
            const float acc = gdg + row_suffix16(dG);
            // the gate a = max(y, lb), y = -A softplus(g + dt_bias): no
            // gradient through the clamped branch; dy/dA_log = y
            const float y2 = -A * U[j];
            const float dy = (live && y2 >= lb2) ? acc : 0.f;
            const float dx = -dy * A * SG[j];
            pa += dy * (y2 * LN2);
            pd[j] = row_sum16(dx);
            vq[j] = dQe + daq * kv[j];
            vk[j] = dKe + dKi + daq * qv[j];
            vg[j] = dx;
            if constexpr (SCALAR) gsum += dx;
        }
        oq[2 * hh] = pack2(vq[0], vq[1]);
        oq[2 * hh + 1] = pack2(vq[2], vq[3]);
        ok[2 * hh] = pack2(vk[0], vk[1]);
        ok[2 * hh + 1] = pack2(vk[2], vk[3]);
        og[2 * hh] = pack2(vg[0], vg[1]);
        og[2 * hh + 1] = pack2(vg[2], vg[3]);
        if (hh == 1) {                                      // both tiles of block kb done
            const int off = (int)((tok * rowe + c0 - 4) * 2);
            __builtin_amdgcn_raw_buffer_store_b128(oq, r_dq, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(ok, r_dk, off, 0, 0);
            if constexpr (!SCALAR) __builtin_amdgcn_raw_buffer_store_b128(og, r_dg, off, 0, 0);
        }
        if (tok == 0) *(f32x4_t *)&part_dtb[sh * PD + c0] = *(const f32x4_t *)&pd[0];
    }
    if (tok == 0) {                                         // channels past the head dimension
#pragma unroll
        for (int kb = NKB; kb < PD / 32; ++kb) {
            float *o = part_dtb + sh * PD + 32 * kb + 8 * grp;
            *(f32x4_t *)&o[0] = zero;
            *(f32x4_t *)&o[4] = zero;
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) pa += __shfl_xor(pa, o, 64);
    if (l == 0) part_alog[sh] = pa;
    if constexpr (SCALAR) {
        gsum += __shfl_xor(gsum, 16, 64);                   // the four lane groups' channels
        gsum += __shfl_xor(gsum, 32, 64);
        if (grp == 0 && live) dgs[(size_t)(t0 + tok) * H + h] = tobf16(gsum);
    }
}

// ---------------------------------------------------------------------------
// prep: one wave per (chunk slot, head), the chunk factors into the two
// scans' bf16 records (in the forward record's MFMA operand layouts,
// RecLayout<KD>, at head dimension KD = 64 or 128):
//   states record (StatesRecT<KD>, kda_bwd_dev.h): Kt and Wm = P^T Kb Gam in the
//     Kt and W^T layouts, and the chunk decay, the operands of
//     X = V - Kt S0 and S1 = Gam S0 + Wm^T X;
//   reverse record: Wm in the Kt layout (the A operand of Wm dS), scale Qt
//     and -Kt in the W^T layout (the A operands of the state-gradient
//     update), scale M^T (the M slot) and the chunk decay.
// The factors are formed as in the chunk kernel: Grams of the rescaled rows
// from (hi, lo) operands, T on fp32 MFMAs, P^T Kb Gam from (hi, lo)
// operands; layouts change through the identity.  The decay regions cover
// 128 channels at either head dimension (zeros past KD).
// ---------------------------------------------------------------------------
template <int KD>
struct PrepWaveLds {
    float beta[CS];
    float dtb[KD];                    // dt_bias in log2 units
    float gam[KD];                    // e^{G_last} per key channel
    float gl[KD];                     // G_last in log2 units
    float tile[CS][CS + 1];           // 16 x 16 transposes
};

template <int KD>
__global__ __launch_bounds__(64) void bwd_prep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ g, const uint16_t *__restrict__ beta,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float lb, float scale,
    const int32_t *__restrict__ cu, int N, int T, int H, uint8_t *__restrict__ srec,
    uint8_t *__restrict__ rrec)
{
    constexpr int NKB = KD / 32, NT = 2 * NKB;
    typedef RecLayout<KD> R;
    typedef StatesRecT<KD> SR;
    __shared__ __attribute__((aligned(16))) PrepWaveLds<KD> L;
    const int64_t slot = blockIdx.x / (unsigned)H;
    const int h = (int)(blockIdx.x % (unsigned)H);
    const int l = threadIdx.x, tok = l & 15, grp = l >> 4;
    const size_t sh = (size_t)slot * H + h;
    int64_t t0;
    const int len = slot_chunk(cu, N, T, slot, t0);
    if (len == 0) return;                                   // gap slot: no scan reads it
    const bool live = tok < len;
    const float A = expf(A_log[h]);
    const float lb2 = lb * LOG2E;
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    const u32x2_t eye = identity_b();
    uint8_t *sr = srec + sh * SR::BYTES;
    uint8_t *rr = rrec + sh * R::BYTES;

    stage_dtb<false, KD>(L.dtb, dt_bias, h, KD);
    IntraInT<NKB> in;
    intra_load<false, KD>(in, q, k, g, beta, t0, len, H, h, KD);
    {
        const float x = bf16f((uint16_t)in.beta);
        const float b = __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * LOG2E));
        if (grp == 0) L.beta[tok] = live ? b : 0.f;
    }
    wave_lds_sync();

    // per channel block: the Grams (rescaled rows), Kt for the states record,
    // scale Qt and -Kt for the reverse record, Kb Gam in the W^T layout
    f32x4_t Akk = zero, AkkT = zero, Aqk = zero;
    u32x2_t kgh[NT], kgl[NT];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        float G[8];
        block_decay<8>(in.g[kb], L.dtb, kb, 0, A, lb2, live, G);
        if (tok == CS - 1) {
            f32x4_t g0, g1, l0, l1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                g0[i] = fast_exp2(G[i]); g1[i] = fast_exp2(G[4 + i]);
                l0[i] = G[i]; l1[i] = G[4 + i];
            }
            *(f32x4_t *)&L.gam[32 * kb + 8 * grp] = g0;
            *(f32x4_t *)&L.gam[32 * kb + 8 * grp + 4] = g1;
            *(f32x4_t *)&L.gl[32 * kb + 8 * grp] = l0;
            *(f32x4_t *)&L.gl[32 * kb + 8 * grp + 4] = l1;
        }
        wave_lds_sync();
        float gl[8];
        *(f32x4_t *)&gl[0] = *(const f32x4_t *)&L.gl[32 * kb + 8 * grp];
        *(f32x4_t *)&gl[4] = *(const f32x4_t *)&L.gl[32 * kb + 8 * grp + 4];
        u32x4_t kth, ktl, qth, qtl, kbh, kbl, kgh4, kgl4, Kh, qs, nk;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            float kt[2], qt[2], kbv[2], kg[2], Kt[2], sq[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * wd + e;
                const float gh = 0.5f * gl[i];
                const float rs = fast_exp2(G[i] - gh), ri = fast_exp2(gh - G[i]);
                const float eg = fast_exp2(G[i]);
                const float kv = elem(in.k[kb], i), qv = elem(in.q[kb], i);
                kt[e] = kv * rs;
                qt[e] = qv * rs;
                kbv[e] = kv * ri;
                kg[e] = kv * fast_exp2(gl[i] - G[i]);
                Kt[e] = kv * eg;
                sq[e] = scale * (qv * eg);
            }
            uint32_t a, b;
            split2(kt[0], kt[1], a, b); kth[wd] = a; ktl[wd] = b;
            split2(qt[0], qt[1], a, b); qth[wd] = a; qtl[wd] = b;
            split2(kbv[0], kbv[1], a, b); kbh[wd] = a; kbl[wd] = b;
            split2(kg[0], kg[1], a, b); kgh4[wd] = a; kgl4[wd] = b;
            Kh[wd] = pack2(Kt[0], Kt[1]);
            qs[wd] = pack2(sq[0], sq[1]);
            nk[wd] = pack2(-Kt[0], -Kt[1]);
        }
        Akk = mm3_k32(kth, ktl, kbh, kbl, Akk);             // Akk[r][c]  = Kt_r . Kb_c
        AkkT = mm3_k32(kbh, kbl, kth, ktl, AkkT);           // AkkT[r][c] = Akk[c][r]
        Aqk = mm3_k32(qth, qtl, kbh, kbl, Aqk);             // Aqk[r][c]  = Qt_r . Kb_c
        __builtin_nontemporal_store(Kh, (u32x4_t *)(sr + SR::KTH + (kb * 64 + l) * 16));
        u32x4_t qw, nw;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int t = 2 * kb + hh;
            const u32x2_t kh2 = {kgh4[2 * hh], kgh4[2 * hh + 1]}, kl2 = {kgl4[2 * hh], kgl4[2 * hh + 1]};
            const u32x2_t q2 = {qs[2 * hh], qs[2 * hh + 1]}, n2 = {nk[2 * hh], nk[2 * hh + 1]};
            kgh[t] = to_wt(kh2, eye);
            kgl[t] = to_wt(kl2, eye);
            const u32x2_t a = to_wt(q2, eye);
            const u32x2_t b = to_wt(n2, eye);
            qw[2 * hh] = a[0]; qw[2 * hh + 1] = a[1];
            nw[2 * hh] = b[0]; nw[2 * hh + 1] = b[1];
        }
        __builtin_nontemporal_store(qw, (u32x4_t *)(rr + R::QT + (kb * 64 + l) * 16));
        __builtin_nontemporal_store(nw, (u32x4_t *)(rr + R::WT + (kb * 64 + l) * 16));
    }
    // the chunk decay into both records, one coalesced store each (128
    // channels, zeros past KD)
    wave_lds_sync();
    {
        const u32x2_t z2 = {0u, 0u};
#pragma unroll
        for (int c = 2 * l; c < SR::GAMC; c += 128) {
            const u32x2_t gv = c < KD ? *(const u32x2_t *)&L.gam[c] : z2;
            __builtin_nontemporal_store(gv, (u32x2_t *)(sr + SR::GAM + c * 4));
            __builtin_nontemporal_store(gv, (u32x2_t *)(rr + R::GAM + c * 4));
        }
    }

    // T = (I + diag(beta) strict_lower(Akk))^-1 as in the chunk kernel
    float br[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) br[j] = L.beta[4 * grp + j];
    const float bc = L.beta[tok];
    f32x4_t Tm;
    {
        f32x4_t N1, N1t, I;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * grp + j;
            N1[j] = tok < r ? -br[j] * Akk[j] : 0.f;
            N1t[j] = r < tok ? -bc * AkkT[j] : 0.f;
            I[j] = r == tok ? 1.f : 0.f;
        }
        const f32x4_t N2 = mm16(N1t, N1), N2t = mm16(N1, N1t);
        const f32x4_t Q12t = mm16(I + N2, I + N1t);
        const f32x4_t N4 = mm16(N2t, N2), N4t = mm16(N2, N2t);
        const f32x4_t Q3t = mm16(I + N4, Q12t);
        const f32x4_t N8 = mm16(N4t, N4);
        Tm = mm16(Q3t, I + N8);
    }
    f32x4_t P, Aq;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        P[j] = Tm[j] * bc;                                  // P = T diag(beta)
        Aq[j] = tok <= 4 * grp + j ? Aqk[j] : 0.f;          // lower_incl(Qt Kb^T)
    }
    {
        // M = Aqk P; the M slot holds scale M^T as an A operand, i.e. scale M
        // in the tile layout
        const f32x4_t M = mm16(tr16(L.tile, Aq), P);
        const u32x2_t mo = {pack2(scale * M[0], scale * M[1]), pack2(scale * M[2], scale * M[3])};
        __builtin_nontemporal_store(mo, (u32x2_t *)(rr + R::M + l * 8));
    }
    // Wm = P^T Kb Gam, tile t in the W^T layout (A = P^T: the tile layout of
    // P), in bf16 for the states record and, through the identity, in the
    // Kt layout for the reverse record
    u32x2_t pAh, pAl;
    split4(P, pAh, pAl);
#pragma unroll
    for (int tp = 0; tp < NKB; ++tp) {
        u32x4_t wh, wk;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int t = 2 * tp + hh;
            const f32x4_t W = mm3_k16(pAh, pAl, kgh[t], kgl[t], zero);
            const u32x2_t a = {pack2(W[0], W[1]), pack2(W[2], W[3])};
            wh[2 * hh] = a[0]; wh[2 * hh + 1] = a[1];
            const f32x4_t d = mfma_k16(a, eye, zero);       // exact: bf16 values
            wk[2 * hh] = pack2(d[0], d[1]);
            wk[2 * hh + 1] = pack2(d[2], d[3]);
        }
        __builtin_nontemporal_store(wh, (u32x4_t *)(sr + SR::WTH + (tp * 64 + l) * 16));
        __builtin_nontemporal_store(wk, (u32x4_t *)(rr + R::KTO + (tp * 64 + l) * 16));
    }
}

// ---------------------------------------------------------------------------
// reduce: per head, the parameter gradients summed over chunk slots in slot
// order (PD = max(K, 128) threads: one channel each; dA_log by a fixed tree).
// ---------------------------------------------------------------------------
template <int PD>
__global__ __launch_bounds__(PD) void bwd_reduce_kernel(
    const float *__restrict__ part_alog, const float *__restrict__ part_dtb, int64_t slots,
    int H, int kd, float *__restrict__ dA_log, float *__restrict__ ddt_bias)
{
    __shared__ float red[PD];
    const int h = blockIdx.x, c = threadIdx.x;
    float s = 0.f, a = 0.f;
    // slot order, sixteen loads issued ahead of their adds
    int64_t sl = 0;
    for (; sl + 16 <= slots; sl += 16) {
        float pv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[i] = part_dtb[((size_t)(sl + i) * H + h) * PD + c];
#pragma unroll
        for (int i = 0; i < 16; ++i) s += pv[i];
    }
    for (; sl < slots; ++sl) s += part_dtb[((size_t)sl * H + h) * PD + c];
    for (int64_t sl = c; sl < slots; sl += PD) a += part_alog[(size_t)sl * H + h];
    if (ddt_bias && c < kd) ddt_bias[(size_t)h * kd + c] = s;
    red[c] = a;
    __syncthreads();
    for (int o = PD / 2; o >= 1; o >>= 1) {
        if (c < o) red[c] += red[c + o];
        __syncthreads();
    }
    if (c == 0) dA_log[h] = red[0];
}

}  // namespace

// One side stream (and its fork / join events) per device, created on first
// use and kept for the life of the process.  The mutex makes each call's
// record / wait / launch sequence on them atomic with respect to other host
// threads.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int MAX_DEVICES = 64;
std::mutex g_side_mutex;
SideStream g_side[MAX_DEVICES];

// The current device's side stream (called with g_side_mutex held).
hipError_t side_stream(SideStream *&out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    SideStream &ss = g_side[dev];
    if (!ss.stream) {
        hipStream_t st = nullptr;
        hipEvent_t a = nullptr, b = nullptr;
        e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&a, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&b, hipEventDisableTiming);
        if (e != hipSuccess) {
            if (b) (void)hipEventDestroy(b);
            if (a) (void)hipEventDestroy(a);
            if (st) (void)hipStreamDestroy(st);
            return e;
        }
        ss.fork = a;
        ss.join = b;
        ss.stream = st;
    }
    out = &ss;
    return hipSuccess;
}

namespace {
// Per (chunk slot, head): the two scans' records, S0 and dS1 (bf16 KD x KD),
// X (bf16 16 x KD), the dt_bias partial sums (max(KD, 128) floats) and the
// A_log partial sum.
template <int KD>
constexpr size_t bwd_slot_bytes() {
    return (size_t)StatesRecT<KD>::BYTES + (size_t)RecLayout<KD>::BYTES +
           (2 * (size_t)KD * KD + (size_t)CS * KD) * sizeof(uint16_t) +
           ((size_t)bwd_pd_stride<KD>() + 1) * sizeof(float);
}
}  // namespace

size_t bwd_workspace_bytes(int64_t num_slots, int H, int K) {
    const size_t sh = (size_t)num_slots * H;
    return sh * (K == 64 ? bwd_slot_bytes<64>() : K == 2 * HD ? bwd_slot_bytes<2 * HD>() : bwd_slot_bytes<HD>());
}

hipError_t launch_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                      const uint16_t *beta, float scale, const float *A_log,
                      const float *dt_bias, float lower_bound, const int32_t *cu, int N, int T,
                      int H, int K, int64_t num_slots, const void *init, int init_fp32,
                      const uint16_t *dout, const float *dfin, uint16_t *dq, uint16_t *dk,
                      uint16_t *dv, uint16_t *dg, uint16_t *dbeta, float *dA_log,
                      float *ddt_bias, float *dinit, void *ws, hipStream_t stream,
                      const hipEvent_t *events, uint16_t *dg_scalar)
{
    const size_t sh = (size_t)num_slots * H;
    // every region starts at a multiple of 256 bytes (each per-(slot, head)
    // size is one, the last region's aside)
    static_assert(RecLayout<HD>::BYTES % 256 == 0 && StatesRecT<HD>::BYTES % 256 == 0 &&
                  RecLayout<64>::BYTES % 256 == 0 && StatesRecT<64>::BYTES % 256 == 0 &&
                  RecLayout<2 * HD>::BYTES % 256 == 0 && StatesRecT<2 * HD>::BYTES % 256 == 0,
                  "256-byte regions");
    const bool k64 = K == 64, k256 = K == 2 * HD;
    const size_t srb = k64 ? StatesRecT<64>::BYTES : k256 ? StatesRecT<2 * HD>::BYTES : StatesRecT<HD>::BYTES;
    const size_t rrb = k64 ? RecLayout<64>::BYTES : k256 ? RecLayout<2 * HD>::BYTES : RecLayout<HD>::BYTES;
    const int pd = k256 ? bwd_pd_stride<2 * HD>() : bwd_pd_stride<HD>();
    uint8_t *srec = (uint8_t *)ws;
    uint8_t *rrec = srec + sh * srb;
    uint16_t *st0 = (uint16_t *)(rrec + sh * rrb);
    uint16_t *dst1 = st0 + sh * K * K;
    uint16_t *xws = dst1 + sh * K * K;
    float *pdtb = (float *)(xws + sh * CS * K);
    float *palog = pdtb + sh * pd;
    const dim3 chunks((unsigned)sh);
    hipError_t e = hipSuccess;
    auto mark = [&](int i) {
        if (events && events[i] && e == hipSuccess) e = hipEventRecord(events[i], stream);
    };
    mark(0);
#define KDA_BWD_PREP(KD_)                                                                     \
    hipLaunchKernelGGL(bwd_prep_kernel<KD_>, chunks, dim3(64), 0, stream,                     \
                       q, k, g, beta, A_log, dt_bias, lower_bound, scale, cu, N, T, H, srec, rrec)
    if (k64) KDA_BWD_PREP(64); else if (k256) KDA_BWD_PREP(2 * HD); else KDA_BWD_PREP(HD);
#undef KDA_BWD_PREP
    mark(1);
    // The reverse scan needs only the prep kernel's records and dO, not the
    // states scan's output: it runs on the device's side stream, forked after
    // prep and joined before the chunk kernel, so that the two
    // latency-bound scans share the compute units.
    if (e == hipSuccess) {
        std::lock_guard<std::mutex> lock(g_side_mutex);
        SideStream *ss = nullptr;
        e = side_stream(ss);
        if (e == hipSuccess) e = hipEventRecord(ss->fork, stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(ss->stream, ss->fork, 0);
        if (e == hipSuccess)
            e = launch_bwd_rscan(dout, rrec, cu, N, T, H, K, dfin, dinit, dv, dst1, ss->stream);
        if (e == hipSuccess) e = hipEventRecord(ss->join, ss->stream);
        if (e == hipSuccess)
            e = launch_bwd_fscan(v, srec, cu, N, T, H, K, init, init_fp32, st0, xws, stream);
        mark(2);
        if (e == hipSuccess) e = hipStreamWaitEvent(stream, ss->join, 0);
    }
    mark(3);
#define KDA_BWD_CHUNK(KD_, SC_)                                                               \
    hipLaunchKernelGGL((bwd_chunk_kernel<KD_, SC_>), chunks, dim3(64), 0, stream, q, k, g, beta, \
                       A_log, dt_bias, lower_bound, scale, dout, cu, N, T, H, st0, dst1, xws, dv, srec, \
                       rrec, dq, dk, dg, dbeta, palog, pdtb, dg_scalar)
    if (dg_scalar) {
        if (k64) KDA_BWD_CHUNK(64, true); else if (k256) KDA_BWD_CHUNK(2 * HD, true); else KDA_BWD_CHUNK(HD, true);
    } else {
        if (k64) KDA_BWD_CHUNK(64, false); else if (k256) KDA_BWD_CHUNK(2 * HD, false); else KDA_BWD_CHUNK(HD, false);
    }
#undef KDA_BWD_CHUNK
    mark(4);
    if (k256)
        hipLaunchKernelGGL(bwd_reduce_kernel<2 * HD>, dim3((unsigned)H), dim3(2 * HD), 0, stream,
                           palog, pdtb, num_slots, H, K, dA_log, ddt_bias);
    else
        hipLaunchKernelGGL(bwd_reduce_kernel<HD>, dim3((unsigned)H), dim3(HD), 0, stream,
                           palog, pdtb, num_slots, H, K, dA_log, ddt_bias);
    mark(5);
    const hipError_t le = hipGetLastError();
    return e != hipSuccess ? e : le;
}

}  // namespace kda
