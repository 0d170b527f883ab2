// Device-side building blocks shared by the libkda kernels (gfx950).
//
// Chunkwise form computed by the kernels (per head, chunk of n <= 16 tokens,
// incoming state S0, in-chunk inclusive cumulative log-decay G):
//   Kt  = k * e^{G},  Qt = q * e^{G},  Kb = k * e^{-G}           (n x 128)
//   T   = (I + diag(beta) strict_lower(Kt Kb^T))^{-1}            (16 x 16)
//   Aqk = lower_incl(Qt Kb^T)
//   M   = Aqk T diag(beta),   W = (T diag(beta))^T Kb diag(e^{G_last})
//                                                                (intra stage)
//   X   = V - Kt S0
//   O   = scale (Qt S0 + M X)
//   S   = diag(e^{G_last}) S0 + W^T X                             (scan)
// With E = T diag(beta) X the usual WY/UT form reads O = Qt S0 + Aqk E and
// S = diag(e^{G_last})(S0 + Kb^T E); folding T diag(beta) (and the chunk
// decay) into M and W moves products off the serial path and lets the intra
// stage round M and W to bf16 once, from fp32 values.  This is the "specialized DPLR"
// chunkwise algorithm the FlashKDA write-up credits for KDA's efficiency
// ("Moonshot AI Open-Sources FlashKDA", section "Why KDA?"), with the
// 16-token chunk and small triangular inverse of its section "What makes
// the kernel fast"; it equals the token recurrence exactly in real
// arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int HD = 128;          // head dimension of the 128-wide tiles (the backward runs K = 64 on them zero-padded)
constexpr int CS = 16;           // tokens per chunk
constexpr int CS_TOKENS = CS;
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Hand-off record written by the intra-chunk stage for one (chunk slot,
// head) and read by the scan.  Every piece is stored in exactly the register
// layout the scan's MFMA operands need.
//
//   KT  [kb 0..3][lane 0..63][8 bf16]  Kt rows as the A operand of a
//        16x16x32 MFMA: lane l holds token l%16, channels 32kb + 8(l/16) + i
//   QT  same for Qt
//   WT  [tp 0..3][lane 0..63][8 bf16]  W^T (decay included) as the A operand of eight
//        16x16x16 MFMAs (state row tiles t = 2tp, 2tp+1): lane l holds
//        channel chan(t, l%16) and tokens 4(l/16) + j, j = 0..3; tile 2tp in
//        bf16 0..3, tile 2tp+1 in bf16 4..7
//   M   [lane][4 bf16]  M as a 16x16x16 A operand (lane l: row l%16,
//        k = 4(l/16) + j)
//   GAM [128 fp32]      e^{G_last} per channel
//
// The state tiles permute their rows so that the accumulator of tile pair
// (2kb, 2kb+1) is directly the B operand of the next chunk's 16x16x32 MFMA:
// row rho of tile t holds channel
//   chan(t, rho) = 32 (t/2) + 8 (rho/4) + 4 (t%2) + rho%4.
// ---------------------------------------------------------------------------
constexpr int REC_KT = 0;
constexpr int REC_QT = 4096;
constexpr int REC_WT = 8192;
constexpr int REC_M = 12288;
constexpr int REC_GAM = 12800;
constexpr int REC_BYTES = 13312;

// The same record for tiles of KT key channels (the head dimension: 64, 128
// or 256): KT/32 channel blocks in KT, QT and WT, KT chunk decays,
// and the whole padded to a multiple of 1 KB (the scan moves records in
// 1 KB DMA units).
template <int KT>
struct RecLayout {
    static_assert(KT == 64 || KT == 128 || KT == 256, "tile widths");
    static constexpr int KTO = 0;
    static constexpr int QT = CS_TOKENS * KT * 2;
    static constexpr int WT = 2 * QT;
    static constexpr int M = 3 * QT;
    static constexpr int GAM = M + CS_TOKENS * CS_TOKENS * 2;
    static constexpr int BYTES = (GAM + KT * 4 + 1023) / 1024 * 1024;
};
static_assert(RecLayout<128>::QT == REC_QT && RecLayout<128>::WT == REC_WT &&
              RecLayout<128>::M == REC_M && RecLayout<128>::GAM == REC_GAM &&
              RecLayout<128>::BYTES == REC_BYTES, "the 128-wide record");

// Record bytes for head dimension K (64, 128 or 256).
__host__ __device__ constexpr int rec_bytes_for(int K) {
    return K > 128 ? RecLayout<256>::BYTES : (K == 64 ? RecLayout<64>::BYTES : RecLayout<128>::BYTES);
}

__host__ __device__ constexpr int state_chan(int t, int rho) {
    return 32 * (t >> 1) + 8 * (rho >> 2) + 4 * (t & 1) + (rho & 3);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t tobf16(float a) {
    __bf16 r = (__bf16)a;
    return __builtin_bit_cast(uint16_t, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// D = A(16x32) B(32x16) + C; lane l supplies A[l%16][8(l/16)+i], B[8(l/16)+i][l%16]
// and holds D[4(l/16)+j][l%16].
__device__ __forceinline__ f32x4_t mfma_k32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// D = A(16x16) B(16x16) + C in bf16; lane l supplies A[l%16][4(l/16)+j], B[4(l/16)+j][l%16].
__device__ __forceinline__ f32x4_t mfma_k16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                     __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}
// D = A(16x4) B(4x16) + C in fp32; lane l supplies A[l%16][l/16], B[l/16][l%16].
__device__ __forceinline__ f32x4_t mfma_k4(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Orders this wave's LDS accesses across its lanes: LDS instructions of one
// wave execute in issue order, so only the compiler must be kept from
// moving accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Raw buffer resource over [p, p + bytes): loads beyond return 0 and stores
// beyond are dropped (checked per dword), which lets partial chunks run
// without branches around memory instructions.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// Sequence n's token range [start, end) in the packed token axis.
__device__ __forceinline__ void seq_range(const int32_t *cu, int n, int T, int64_t &start, int64_t &end) {
    if (cu) { start = cu[n]; end = cu[n + 1]; }
    else { start = (int64_t)n * T; end = start + T; }
}

// First chunk slot of sequence n: floor(start / 16) + n.  Slots of
// consecutive sequences never overlap and all lie below floor(total/16) + N.
__device__ __forceinline__ int64_t seq_slot0(const int32_t *cu, int n, int T) {
    int64_t s = cu ? (int64_t)cu[n] : (int64_t)n * T;
    return s / CS + n;
}

}  // namespace kda
