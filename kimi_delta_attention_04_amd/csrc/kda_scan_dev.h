// Building blocks of the scan kernels (kda_scan.hip, kda_bwd_scan.hip):
// the LDS ring that the DMA wave fills with each chunk's record and token
// tile, the explicit vmcnt / barrier waits of its protocol, and the chunk
// decay applied to the state tiles held in MFMA accumulators.
#pragma once

#include "kda_device.h"

namespace kda {

namespace {

// LDS ring slots per workgroup (chunks in flight + the one being read); the
// DMA wave's vmcnt (at most 63) must cover DEPTH-1 chunks of DMAs.
template <int CW> constexpr int RING_DEPTH = CW <= 64 ? 5 : 4;
// One operand set in registers (head dimension 256, or two slices per
// wave): the operands are read one chunk at a time (no operand prefetch, see
// scan_kernel), so the vmcnt covers DEPTH-2 chunks of DMAs.
constexpr int RING_DEPTH_256 = 4;
constexpr int REC_KB = REC_BYTES / 1024;         // 13 one-kilobyte units per record

static_assert(REC_BYTES % 1024 == 0, "record must be a whole number of 1 KB units");
static_assert(RecLayout<256>::BYTES % 1024 == 0, "record must be a whole number of 1 KB units");

// s_waitcnt vmcnt(n) followed by a workgroup barrier; waits for this wave's
// LDS traffic too but, unlike __syncthreads(), not for every outstanding
// global access.
template <int NV>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(NV >= 0 && NV <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(NV) : "memory");
}

// Workgroup barrier after this wave's LDS accesses have completed (its
// global stores may still be in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Raw buffer descriptor words (base, stride 0, num_records, the same
// configuration word as make_rsrc) for the inline-assembly DMA below.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t rsrc_words(const void *p, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    i32x4_t r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}

// 16-byte-per-lane buffer-to-LDS DMA: lane l's 16 bytes at byte offset `off`
// of the resource land at LDS address lds + 16 l.  Issued from inline
// assembly so that the compiler's own wait insertion, which cannot tell the
// ring slots apart, does not serialise the prefetch; the waits are explicit
// (wait_vm_barrier).  The loop that uses it issues no other loads.  m0 (the
// LDS address of the DMA) is set by the asm itself and declared clobbered.
__device__ __forceinline__ void dma16(i32x4_t rs, const void *lds, int off) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(off), "s"(rs) : "memory", "m0");
}

template <int CW, int RB = REC_BYTES>
struct alignas(16) ScanSlot {
    uint8_t rec[RB];
    uint16_t v[CS][CW];
};

// Lane n of each 16-lane row, broadcast to the whole row (DPP row_newbcast);
// the compiler folds it into the consuming VALU instruction.
template <int SRC>
__device__ __forceinline__ float row_bcast(float x) {
    static_assert(SRC >= 0 && SRC < 16, "row lane");
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                              0x150 + SRC, 0xf, 0xf, true));
}

// The MFMA operands of one chunk, as one wave holds them in registers.
// NKB 32-channel blocks of the key dimension (4, or 8 for head dimension 256).
template <int CT, int NKB = 4>
struct ChunkOps {
    u32x4_t kt[NKB], qt[NKB], wt[NKB];
    u32x2_t m;
    float gm[NKB >= 4 ? NKB / 2 : 2];   // chunk decay of two state rows per 128 channels (see load_ops)
    u32x2_t v[CT];            // v[row l%16][4(l/16) .. +3] of each slice: an MFMA A operand
};

// Row multiplier of the decay: S[t][j] (state row chan(t, 4grp + j)) takes
// the chunk decay that lane 4(t'/2) + 2(t'%2) + j/2 of its 16-lane row holds
// in gm[2(t/8) + j%2], t' = t % 8.  Lane cg of row grp loads the decays of
// channels 128p + 32(cg/4) + 8grp + 4((cg/2)%2) + 2(cg%2) + {0, 1} into
// gm[2p], gm[2p+1], which is exactly that.
template <int T, int J, int NG>
__device__ __forceinline__ float decay_of(const float (&gm)[NG]) {
    constexpr int TT = T & 7;
    return row_bcast<4 * (TT >> 1) + 2 * (TT & 1) + (J >> 1)>(gm[2 * (T >> 3) + (J & 1)]);
}

// S[t] *= diag(chunk decay) for the state row tiles t = T .. NT-1.
template <int T, int NT, int NG>
__device__ __forceinline__ void decay_tiles(f32x4_t (&S)[NT], const float (&gm)[NG]) {
    if constexpr (T < NT) {
        S[T][0] *= decay_of<T, 0>(gm);
        S[T][1] *= decay_of<T, 1>(gm);
        S[T][2] *= decay_of<T, 2>(gm);
        S[T][3] *= decay_of<T, 3>(gm);
        decay_tiles<T + 1, NT>(S, gm);
    }
}

}  // namespace

// Compute units of the current device (cached per device).
int num_cus();

}  // namespace kda
