// Inter-chunk scan: the sequential part of the chunkwise algorithm.
//
// A workgroup owns one (sequence, head, column part); each of its NW compute
// waves (four, or two when a head is split over four workgroups) keeps CT
// 16-column slices of the 128-row (256-row at head dimension 256) fp32 state
// in MFMA accumulators for the whole sequence.  Columns of the state evolve independently (each
// sees the same transition and its own v entries), so column parts need no
// communication.  The row permutation of the state tiles (kda_device.h)
// makes the accumulators of tile pair (2kb, 2kb+1), rounded to bf16, exactly
// the B operand of the next chunk's 16x16x32 MFMAs: the state never leaves
// the registers.  Per chunk:
//   P = Kt S,  X = V - P,  O = scale (Qt S + M X) -> bf16,  S = W^T X + diag(gamma) S
// (W carries the chunk decay, so diag(gamma) S is formed while the P
// products run and enters the update MFMAs as their accumulator).
//
// The hand-off record of each chunk (13 KB, 26 KB at head dimension 256)
// and the chunk's v tile are read from memory once per workgroup, by
// buffer-to-LDS DMA into a ring of DEPTH slots, DEPTH-1 chunks ahead of the
// compute.  One more wave issues
// all of the DMAs; the compute waves read their MFMA operands from the ring
// and never wait on the DMA themselves.  Every memory access goes
// through a range-checked buffer resource, so partial chunks need no
// branches and the number of DMAs per chunk is fixed, which is what the
// DMA wave's explicit vmcnt accounting relies on.  The serial chain is what
// the FlashKDA write-up calls the low-parallelism second stage ("Moonshot AI
// Open-Sources FlashKDA", section "What makes the kernel fast").
#include "kda_device.h"
#include "kda_launch.h"

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
    float gm[NKB / 2];        // chunk decay of two state rows per 128 channels (see load_ops)
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

// CT 16-column slices per compute wave, NW compute waves (and the DMA wave)
// per workgroup; head dimension K = V = VD (128, 256, or 64 on the 128-wide
// tiles).
//
// Two ring protocols.  One slice per wave on 128-wide tiles: the compute
// waves read chunk c+1's operands into registers while they compute chunk c
// (two operand sets in registers).  256-wide tiles, and two slices per wave:
// one operand set (at 256, 96 registers for Kt, Qt and W^T alone; with two
// slices per wave, so that 168 registers let two workgroups share a CU), so
// the compute waves read chunk c's operands at the top of its own
// iteration, and the DMA wave refills the slot of chunk c-1 instead of
// chunk c's.  The second launch-bounds argument is the minimum number of
// waves per SIMD the register allocation must allow.
template <int CT, int NW, int VD>
__global__ __launch_bounds__(64 * (NW + 1), VD > HD ? 1 : (CT == 2 ? 3 : 2)) void scan_kernel(
    const uint16_t *__restrict__ v, const uint8_t *__restrict__ ws,
    const int32_t *__restrict__ cu, int N, int T, int H, float scale,
    const void *__restrict__ init, int init_fp32,
    void *__restrict__ fin, int fin_fp32, uint16_t *__restrict__ out)
{
    constexpr int CW = NW * 16 * CT;                 // columns per workgroup
    constexpr int K = VD, V = VD;
    constexpr bool WIDE = VD > HD;                   // 256-wide tiles
    constexpr int KTL = WIDE ? 2 * HD : HD;          // key channels of the tiles
    constexpr int NT = KTL / 16;                     // state row tiles per slice
    constexpr int NKB = KTL / 32;                    // 32-channel blocks
    typedef RecLayout<KTL> R;
    constexpr int RKB = R::BYTES / 1024;             // one-kilobyte units per record
    constexpr int NSPLIT = V / CW;                   // column parts per head
    static_assert(NSPLIT * CW == V, "column parts cover the head");
    constexpr int V_KB = CS * CW * 2 / 1024;         // one-kilobyte units of a v tile
    constexpr int UNITS = RKB + V_KB;                // DMA units per chunk
    constexpr int VROW_LANES = CW * 2 / 16;          // lanes per v row in a DMA unit
    // one operand set in registers (the protocol of 256-wide tiles) also for
    // two slices per wave, so that two workgroups fit a CU's register file
    constexpr bool ONESET = WIDE || CT == 2;
    constexpr int DEPTH = ONESET ? RING_DEPTH_256 : RING_DEPTH<CW>;
    __shared__ ScanSlot<CW, R::BYTES> ring[DEPTH];
    static_assert((DEPTH - (ONESET ? 2 : 1)) * UNITS <= 63, "vmcnt holds at most 63");

    // Block b -> (unit u, part): the parts of a unit share b mod 8 (same XCD, same L2).
    const int b = blockIdx.x;
    const int u = 8 * (b / (8 * NSPLIT)) + (b & 7);
    const int part = (b >> 3) % NSPLIT;
    if (u >= N * H) return;                           // block-uniform
    const int n = u / H, h = u % H;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int l = tid & 63;
    const int grp = l >> 4, cg = l & 15;
    const bool dma_wave = w == NW;                    // the wave that issues the ring DMAs
    const int wcol0 = (dma_wave ? 0 : w) * 16 * CT;   // first column of this wave within the part
    const int col0 = part * CW;                       // first column of the part within the head

    int64_t start, end;
    seq_range(cu, n, T, start, end);
    const int64_t L = end - start;
    const int nch = (int)((L + CS - 1) / CS);
    const int64_t slot0 = seq_slot0(cu, n, T);
    // K = V = 128 or 256, or 64 on the 128-wide tiles: state rows from K on stay zero
    // (they load as zeros from the range-checked state buffers, receive no
    // updates since their key channels are zero, and are not stored)
    const size_t row_bytes = (size_t)H * V * 2;       // one token row of v / out

    // ---- state slices: S[ct][t][j] = state[chan(t, 4grp+j)][col] -------------
    // (a zero-sized resource when there is no initial state: loads return 0)
    f32x4_t S[CT][NT];
    if (!dma_wave) {
        const size_t slab = (size_t)K * V * (init_fp32 ? 4 : 2);
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc((const uint8_t *)init + (init ? ((size_t)n * H + h) * slab : 0),
                      init ? (uint32_t)slab : 0u);
        if (init_fp32) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int idx = state_chan(t, 4 * grp + j) * V + col0 + wcol0 + 16 * ct + cg;
                        S[ct][t][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, idx * 4, 0, 0));
                    }
        } else {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int idx = state_chan(t, 4 * grp + j) * V + col0 + wcol0 + 16 * ct + cg;
                        S[ct][t][j] = bf16f(__builtin_amdgcn_raw_buffer_load_b16(rs, idx * 2, 0, 0));
                    }
        }
    }
    // state loads complete before the DMA accounting starts
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Per-chunk addressing advances by fixed strides.
    const size_t rec_stride = (size_t)H * R::BYTES;
    const size_t row_stride = (size_t)CS * H * V;                  // elements per chunk of v / out
    const uint8_t *rec_base = ws + ((size_t)slot0 * H + h) * R::BYTES;
    const uint16_t *v_base = v + ((size_t)start * H + h) * V + col0;
    uint16_t *out_base = out + ((size_t)start * H + h) * V + col0;

    // Chunk c -> ring slot c % DEPTH by DMA (DMA wave): unit k < RKB is
    // kilobyte k of the record; the next V_KB units are the v tile of this
    // part, one row of CW columns per VROW_LANES lanes (rows past the sequence
    // end and chunks past the last one read as zeros).  Exactly UNITS DMAs
    // per chunk.
    auto issue = [&](int c, int slot) {
        const bool live = c < nch;
        const i32x4_t rr =
            rsrc_words(rec_base + (live ? (size_t)c * rec_stride : 0), live ? (uint32_t)R::BYTES : 0u);
        const int64_t rem = L - (int64_t)c * CS;
        const int len = live ? (int)(rem < CS ? rem : CS) : 0;
        const i32x4_t rv =
            rsrc_words(v_base + (live ? (size_t)c * row_stride : 0), (uint32_t)(len * row_bytes));
        ScanSlot<CW, R::BYTES> &sl = ring[slot];
#pragma unroll
        for (int unit = 0; unit < RKB; ++unit) dma16(rr, &sl.rec[unit * 1024], unit * 1024 + l * 16);
#pragma unroll
        for (int vu = 0; vu < V_KB; ++vu) {
            const int vrow0 = vu * (1024 / (2 * CW));                  // 1 KB = 1024 / (2 CW) rows
            dma16(rv, &sl.v[vrow0][0],
                  (int)((vrow0 + l / VROW_LANES) * row_bytes) + (l % VROW_LANES) * 16);
        }
    };

    // LDS -> registers: the operands of the chunk in ring slot `slot`.
    auto load_ops = [&](int slot, ChunkOps<CT, NKB> &op) {
        const ScanSlot<CW, R::BYTES> &sl = ring[slot];
        const uint8_t *Rp = sl.rec;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            op.kt[kb] = *(const u32x4_t *)(Rp + R::KTO + (kb * 64 + l) * 16);
            op.qt[kb] = *(const u32x4_t *)(Rp + R::QT + (kb * 64 + l) * 16);
            op.wt[kb] = *(const u32x4_t *)(Rp + R::WT + (kb * 64 + l) * 16);
        }
        op.m = *(const u32x2_t *)(Rp + R::M + l * 8);
        const int gch = 32 * (cg >> 2) + 8 * grp + 4 * ((cg >> 1) & 1) + 2 * (cg & 1);
#pragma unroll
        for (int p = 0; p < NKB / 4; ++p) {
            const u32x2_t g2 = *(const u32x2_t *)(Rp + R::GAM + (128 * p + gch) * 4);
            op.gm[2 * p] = __uint_as_float(g2[0]);
            op.gm[2 * p + 1] = __uint_as_float(g2[1]);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
            op.v[ct] = *(const u32x2_t *)&sl.v[cg][wcol0 + 16 * ct + 4 * grp];
    };

    // Identity as a 16x16x16 B operand (lane l: k = 4(l/16) + j, column l%16):
    // D = A I moves a tile from the A-operand layout to the accumulator
    // layout, exactly for bf16 data.
    u32x2_t eye;
    {
        const uint32_t one = 0x3f80u;                 // bf16 1.0
        const int d = cg - 4 * grp;
        eye[0] = (d == 0 ? one : 0u) | (d == 1 ? one << 16 : 0u);
        eye[1] = (d == 2 ? one : 0u) | (d == 3 ? one << 16 : 0u);
    }
    auto compute = [&](int c, const ChunkOps<CT, NKB> &op) {
        const int64_t rem = L - (int64_t)c * CS;
        const int len = (int)(rem < CS ? rem : CS);
        // rows past the sequence end fall outside the resource and are dropped
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(out_base + (size_t)c * row_stride, (uint32_t)((len - 1) * row_bytes + CW * 2));
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int lc = wcol0 + 16 * ct + cg;         // column within the part
            // bf16 copy of the state as B operand: k-slots 8grp..8grp+7 of pair kb
            u32x4_t Sb[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                Sb[kb][0] = pack2(S[ct][2 * kb][0], S[ct][2 * kb][1]);
                Sb[kb][1] = pack2(S[ct][2 * kb][2], S[ct][2 * kb][3]);
                Sb[kb][2] = pack2(S[ct][2 * kb + 1][0], S[ct][2 * kb + 1][1]);
                Sb[kb][3] = pack2(S[ct][2 * kb + 1][2], S[ct][2 * kb + 1][3]);
            }
            // P in two independent halves (a shorter dependent MFMA chain on
            // the serial path); v into the accumulator layout
            f32x4_t P0 = zero, P1 = zero, Qs = zero;
#pragma unroll
            for (int i = 0; i < NKB / 2; ++i) {
                P0 = mfma_k32(op.kt[i], Sb[i], P0);
                P1 = mfma_k32(op.kt[NKB / 2 + i], Sb[NKB / 2 + i], P1);
            }
            const f32x4_t vv = mfma_k16(op.v[ct], eye, zero);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) Qs = mfma_k32(op.qt[kb], Sb[kb], Qs);
            // decayed old state: the accumulator the update MFMAs add W^T X to
            decay_tiles<0, NT>(S[ct], op.gm);
            u32x2_t Xb;
            Xb[0] = pack2(vv[0] - (P0[0] + P1[0]), vv[1] - (P0[1] + P1[1]));
            Xb[1] = pack2(vv[2] - (P0[2] + P1[2]), vv[3] - (P0[3] + P1[3]));
#pragma unroll
            for (int tp = 0; tp < NKB; ++tp) {
                u32x2_t lo = {op.wt[tp][0], op.wt[tp][1]}, hi = {op.wt[tp][2], op.wt[tp][3]};
                S[ct][2 * tp] = mfma_k16(lo, Xb, S[ct][2 * tp]);
                S[ct][2 * tp + 1] = mfma_k16(hi, Xb, S[ct][2 * tp + 1]);
            }
            // M X in an accumulator of its own (no accumulator chaining
            // between MFMA opcodes of different shapes), added on the VALU
            const f32x4_t MX = mfma_k16(op.m, Xb, zero);
            // O^T through the identity: lane (grp, cg) then holds token cg,
            // columns 4grp .. 4grp+3 of the slice, one 8-byte store
            const u32x2_t oa = {pack2(scale * (Qs[0] + MX[0]), scale * (Qs[1] + MX[1])),
                                pack2(scale * (Qs[2] + MX[2]), scale * (Qs[3] + MX[3]))};
            const f32x4_t ot = mfma_k16(oa, eye, zero);
            const u32x2_t os = {pack2(ot[0], ot[1]), pack2(ot[2], ot[3])};
            __builtin_amdgcn_raw_buffer_store_b64(os, ro, (int)(cg * row_bytes) + (lc - cg + 4 * grp) * 2, 0, 0);
        }
    };

    // Software pipeline.  Iteration c: the DMA wave waits for chunk c+1 to
    // land, the compute waves finish their reads of chunk c (issued in
    // iteration c-1), all the waves meet at a barrier; then the compute waves
    // read chunk c+1 into registers and compute chunk c while the DMA wave
    // refills chunk c's slot with chunk c+DEPTH.  The DMA wave issues chunks
    // in order, UNITS DMAs each, so at the top of iteration c the DMAs issued
    // after chunk c+1's number (DEPTH-2) UNITS (and (DEPTH-1) UNITS after
    // chunk 0's before the first iteration).
    if constexpr (ONESET) {
        // One operand set (256-wide tiles, or two slices per wave).  Iteration c: the DMA wave waits for chunk c to
        // land, the compute waves finish their reads of chunk c-1, all the
        // waves meet at a barrier; then the compute waves read chunk c and
        // compute it while the DMA wave refills chunk c-1's slot with chunk
        // c-1+DEPTH.  DEPTH-1 chunks are issued before the first iteration,
        // so at the top of iteration c the DMAs issued after chunk c's number
        // (DEPTH-2) UNITS.
        if (dma_wave) {
#pragma unroll
            for (int c = 0; c < DEPTH - 1; ++c) issue(c, c);
            int slot = DEPTH - 1;                    // ring slot of chunk c-1
            for (int c = 0; c < nch; ++c) {
                wait_vm_barrier<(DEPTH - 2) * UNITS>();  // chunk c landed; slot of c-1 free
                issue(c - 1 + DEPTH, slot);
                slot = slot == DEPTH - 1 ? 0 : slot + 1;
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            return;
        }
        ChunkOps<CT, NKB> op;
        int cur = 0;                                 // ring slot of chunk c
        for (int c = 0; c < nch; ++c) {
            lds_barrier();                           // own reads of chunk c-1 done; chunk c landed
            load_ops(cur, op);
            compute(c, op);
            cur = cur == DEPTH - 1 ? 0 : cur + 1;
        }
    } else {
    if (dma_wave) {
#pragma unroll
        for (int c = 0; c < DEPTH; ++c) issue(c, c);
        wait_vm_barrier<(DEPTH - 1) * UNITS>();      // chunk 0 landed
        int slot = 0;
        for (int c = 0; c < nch; ++c) {
            wait_vm_barrier<(DEPTH - 2) * UNITS>();  // chunk c+1 landed; slot of c free
            issue(c + DEPTH, slot);
            slot = slot == DEPTH - 1 ? 0 : slot + 1;
        }
        // drain the DMAs of the chunks past the end before the workgroup exits
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }
    lds_barrier();                                   // chunk 0 landed

    ChunkOps<CT, NKB> opA, opB;
    load_ops(0, opA);
    int next = 1;                                     // ring slot of chunk c+1
    auto step = [&](int c, const ChunkOps<CT, NKB> &cur, ChunkOps<CT, NKB> &nxt) {
        lds_barrier();                               // own reads of chunk c done; chunk c+1 landed
        load_ops(next, nxt);
        compute(c, cur);
        next = next == DEPTH - 1 ? 0 : next + 1;
    };
    for (int c = 0; c < nch; c += 2) {
        step(c, opA, opB);
        if (c + 1 < nch) step(c + 1, opB, opA);
    }
    }

    if (fin) {
        const size_t slab = (size_t)K * V * (fin_fp32 ? 4 : 2);
        const __amdgpu_buffer_rsrc_t rf =
            make_rsrc((uint8_t *)fin + ((size_t)n * H + h) * slab, (uint32_t)slab);
        if (fin_fp32) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int idx = state_chan(t, 4 * grp + j) * V + col0 + wcol0 + 16 * ct + cg;
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[ct][t][j]), rf, idx * 4, 0, 0);
                    }
        } else {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int idx = state_chan(t, 4 * grp + j) * V + col0 + wcol0 + 16 * ct + cg;
                        __builtin_amdgcn_raw_buffer_store_b16(tobf16(S[ct][t][j]), rf, idx * 2, 0, 0);
                    }
        }
    }
}

// Reverse scan of the backward pass: the state gradient dS (key channels x
// value columns) of one (sequence, head), chunk by chunk from the last, on
// the forward scan's structure (each compute wave one 16-column slice in
// MFMA accumulators, the records and the d_out tiles arriving in an LDS ring
// by DMA from a wave of their own, one barrier per chunk).  With dS1 the
// gradient reaching the chunk's end state (the kernel's dfin for the last
// chunk):
//   dX = Wm dS1 + scale M^T dO,   dV = dX
//   dS0 = diag(gamma) dS1 + scale Qt^T dO - Kt^T dX
// (the chain rule through the chunk step O = scale (Qt S0 + M X),
// S1 = diag(gamma) S0 + Wm^T X, X = V - Kt S0).  The record of each chunk
// (written by the backward's prep kernel) holds Wm in the Kt slot, scale Qt
// and -Kt transposed in the Qt and W^T slots, scale M^T in the M slot.
// Stored per chunk for the chunk kernel: dS1 rounded to bf16, as rows of
// each 16-column part ([part][row][16 columns]), and dX in fp32 ([16][V]).
// One slice per wave on the 128-wide tiles (K = V = 128, or 64 with V = 64
// columns and the rows from 64 on zero).
template <int NW, int VD>
__global__ __launch_bounds__(64 * (NW + 1), NW > 4 ? 1 : 2) void rscan_kernel(
    const uint16_t *__restrict__ dout, const uint8_t *__restrict__ rrec,
    const int32_t *__restrict__ cu, int N, int T, int H,
    const float *__restrict__ dfin, float *__restrict__ dinit, uint16_t *__restrict__ dv,
    uint16_t *__restrict__ ds1)
{
    constexpr int CW = NW * 16;
    constexpr int V = VD;
    constexpr int NT = HD / 16, NKB = HD / 32;
    typedef RecLayout<HD> R;
    constexpr int RKB = R::BYTES / 1024;
    constexpr int NSPLIT = V / CW;
    static_assert(NSPLIT * CW == V, "column parts cover the head");
    constexpr int V_KB = CS * CW * 2 / 1024;
    constexpr int UNITS = RKB + V_KB;
    constexpr int VROW_LANES = CW * 2 / 16;
    constexpr int DEPTH = RING_DEPTH<CW>;
    __shared__ ScanSlot<CW, R::BYTES> ring[DEPTH];
    static_assert((DEPTH - 1) * UNITS <= 63, "vmcnt holds at most 63");

    const int b = blockIdx.x;
    const int u = 8 * (b / (8 * NSPLIT)) + (b & 7);
    const int part = (b >> 3) % NSPLIT;
    if (u >= N * H) return;                           // block-uniform
    const int n = u / H, h = u % H;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int grp = l >> 4, cg = l & 15;
    const bool dma_wave = w == NW;
    const int wcol0 = (dma_wave ? 0 : w) * 16;
    const int col0 = part * CW;
    const int p16 = (col0 + wcol0) >> 4;              // this wave's 16-column part of the head

    int64_t start, end;
    seq_range(cu, n, T, start, end);
    const int64_t L = end - start;
    const int nch = (int)((L + CS - 1) / CS);
    const int64_t slot0 = seq_slot0(cu, n, T);
    const size_t row_bytes = (size_t)H * V * 2;

    f32x4_t S[NT];
    if (!dma_wave) {
        const size_t slab = (size_t)V * V * 4;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc((const uint8_t *)dfin + (dfin ? ((size_t)n * H + h) * slab : 0), dfin ? (uint32_t)slab : 0u);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = state_chan(t, 4 * grp + j);
                const int idx = row * V + col0 + wcol0 + cg;
                S[t][j] = row < V ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, idx * 4, 0, 0)) : 0.f;
            }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const size_t rec_stride = (size_t)H * R::BYTES;
    const size_t row_stride = (size_t)CS * H * V;
    const uint8_t *rec_base = rrec + ((size_t)slot0 * H + h) * R::BYTES;
    const uint16_t *d_base = dout + ((size_t)start * H + h) * V + col0;
    uint16_t *dv_base = dv + ((size_t)start * H + h) * V + col0;

    // iteration c handles chunk nch - 1 - c; DMA units as in scan_kernel
    auto issue = [&](int c, int slot) {
        const bool live = c < nch;
        const int ci = live ? nch - 1 - c : 0;
        const i32x4_t rr =
            rsrc_words(rec_base + (size_t)ci * rec_stride, live ? (uint32_t)R::BYTES : 0u);
        const int64_t rem = L - (int64_t)ci * CS;
        const int len = live ? (int)(rem < CS ? rem : CS) : 0;
        const i32x4_t rv = rsrc_words(d_base + (size_t)ci * row_stride, (uint32_t)(len * row_bytes));
        ScanSlot<CW, R::BYTES> &sl = ring[slot];
#pragma unroll
        for (int unit = 0; unit < RKB; ++unit) dma16(rr, &sl.rec[unit * 1024], unit * 1024 + l * 16);
#pragma unroll
        for (int vu = 0; vu < V_KB; ++vu) {
            const int vrow0 = vu * (1024 / (2 * CW));
            dma16(rv, &sl.v[vrow0][0], (int)((vrow0 + l / VROW_LANES) * row_bytes) + (l % VROW_LANES) * 16);
        }
    };
    auto load_ops = [&](int slot, ChunkOps<1, NKB> &op) {
        const ScanSlot<CW, R::BYTES> &sl = ring[slot];
        const uint8_t *Rp = sl.rec;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            op.kt[kb] = *(const u32x4_t *)(Rp + R::KTO + (kb * 64 + l) * 16);
            op.qt[kb] = *(const u32x4_t *)(Rp + R::QT + (kb * 64 + l) * 16);
            op.wt[kb] = *(const u32x4_t *)(Rp + R::WT + (kb * 64 + l) * 16);
        }
        op.m = *(const u32x2_t *)(Rp + R::M + l * 8);
        const int gch = 32 * (cg >> 2) + 8 * grp + 4 * ((cg >> 1) & 1) + 2 * (cg & 1);
        const u32x2_t g2 = *(const u32x2_t *)(Rp + R::GAM + gch * 4);
        op.gm[0] = __uint_as_float(g2[0]);
        op.gm[1] = __uint_as_float(g2[1]);
        op.v[0] = *(const u32x2_t *)&sl.v[cg][wcol0 + 4 * grp];
    };
    u32x2_t eye;
    {
        const uint32_t one = 0x3f80u;
        const int d = cg - 4 * grp;
        eye[0] = (d == 0 ? one : 0u) | (d == 1 ? one << 16 : 0u);
        eye[1] = (d == 2 ? one : 0u) | (d == 3 ? one << 16 : 0u);
    }
    auto compute = [&](int c, const ChunkOps<1, NKB> &op) {
        const int ci = nch - 1 - c;
        const int64_t rem = L - (int64_t)ci * CS;
        const int len = (int)(rem < CS ? rem : CS);
        const size_t sh = (size_t)(slot0 + ci) * H + h;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        // bf16 copy of dS1: the B operand of Wm dS1, and the stored dS1
        u32x4_t Sb[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            Sb[kb][0] = pack2(S[2 * kb][0], S[2 * kb][1]);
            Sb[kb][1] = pack2(S[2 * kb][2], S[2 * kb][3]);
            Sb[kb][2] = pack2(S[2 * kb + 1][0], S[2 * kb + 1][1]);
            Sb[kb][3] = pack2(S[2 * kb + 1][2], S[2 * kb + 1][3]);
        }
        f32x4_t P0 = zero, P1 = zero;
#pragma unroll
        for (int i = 0; i < NKB / 2; ++i) {
            P0 = mfma_k32(op.kt[i], Sb[i], P0);
            P1 = mfma_k32(op.kt[NKB / 2 + i], Sb[NKB / 2 + i], P1);
        }
        // dO into the accumulator layout (tokens 4grp + j of column cg), then
        // as the k = 16 B operand; scale M^T dO
        const f32x4_t dd = mfma_k16(op.v[0], eye, zero);
        const u32x2_t dOb = {pack2(dd[0], dd[1]), pack2(dd[2], dd[3])};
        const f32x4_t MdO = mfma_k16(op.m, dOb, zero);
        decay_tiles<0, NT>(S, op.gm);
        f32x4_t dX;
#pragma unroll
        for (int j = 0; j < 4; ++j) dX[j] = (P0[j] + P1[j]) + MdO[j];
        const u32x2_t dXb = {pack2(dX[0], dX[1]), pack2(dX[2], dX[3])};
#pragma unroll
        for (int tp = 0; tp < NKB; ++tp) {
            const u32x2_t qlo = {op.qt[tp][0], op.qt[tp][1]}, qhi = {op.qt[tp][2], op.qt[tp][3]};
            const u32x2_t klo = {op.wt[tp][0], op.wt[tp][1]}, khi = {op.wt[tp][2], op.wt[tp][3]};
            S[2 * tp] = mfma_k16(qlo, dOb, S[2 * tp]);
            S[2 * tp + 1] = mfma_k16(qhi, dOb, S[2 * tp + 1]);
            S[2 * tp] = mfma_k16(klo, dXb, S[2 * tp]);
            S[2 * tp + 1] = mfma_k16(khi, dXb, S[2 * tp + 1]);
        }
        // stores (off the chain): dV = dX in bf16 through the identity (lane
        // (grp, cg): token cg, columns 4grp .. +3), which the chunk kernel
        // also takes as dX, and dS1 in bf16 as rows (the identity turns tile
        // t into lane (grp, cg): state row chan(t, cg), columns 4grp .. +3 of
        // the slice)
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(dv_base + (size_t)ci * row_stride, (uint32_t)((len - 1) * row_bytes + CW * 2));
        const f32x4_t vt = mfma_k16(dXb, eye, zero);
        const u32x2_t vs = {pack2(vt[0], vt[1]), pack2(vt[2], vt[3])};
        __builtin_amdgcn_raw_buffer_store_b64(vs, ro, (int)(cg * row_bytes) + (wcol0 + 4 * grp) * 2, 0, 0);
        uint16_t *so = ds1 + sh * HD * HD + (size_t)p16 * HD * 16 + 4 * grp;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const u32x2_t a = {Sb[t >> 1][2 * (t & 1)], Sb[t >> 1][2 * (t & 1) + 1]};
            const f32x4_t st = mfma_k16(a, eye, zero);
            const u32x2_t sv = {pack2(st[0], st[1]), pack2(st[2], st[3])};
            *(u32x2_t *)&so[state_chan(t, cg) * 16] = sv;
        }
    };

    // the two-operand-set protocol of scan_kernel
    if (dma_wave) {
#pragma unroll
        for (int c = 0; c < DEPTH; ++c) issue(c, c);
        wait_vm_barrier<(DEPTH - 1) * UNITS>();
        int slot = 0;
        for (int c = 0; c < nch; ++c) {
            wait_vm_barrier<(DEPTH - 2) * UNITS>();
            issue(c + DEPTH, slot);
            slot = slot == DEPTH - 1 ? 0 : slot + 1;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }
    lds_barrier();
    ChunkOps<1, NKB> opA, opB;
    load_ops(0, opA);
    int next = 1;
    auto step = [&](int c, const ChunkOps<1, NKB> &cur, ChunkOps<1, NKB> &nxt) {
        lds_barrier();
        load_ops(next, nxt);
        compute(c, cur);
        next = next == DEPTH - 1 ? 0 : next + 1;
    };
    for (int c = 0; c < nch; c += 2) {
        step(c, opA, opB);
        if (c + 1 < nch) step(c + 1, opB, opA);
    }
    if (dinit) {
        const size_t base = ((size_t)n * H + h) * V * V;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = state_chan(t, 4 * grp + j);
                if (row < V) dinit[base + (size_t)row * V + col0 + wcol0 + cg] = S[t][j];
            }
    }
}

// Forward scan of the backward pass: the state S of one (sequence, head)
// from the initial state through every chunk (X = V - Kt S0,
// S1 = diag(gamma) S0 + Wm^T X, with the state and X as (hi, lo) bf16
// operands), without the output, storing
// per chunk for the chunk kernel the start state S0 rounded to bf16 (rows of
// each 16-column part, [part][128 rows][16 columns]) and X in fp32
// ([16][V]).  The record of each chunk (written by the backward's prep
// kernel) holds Kt and Wm in the forward record's Kt and W^T slots and the
// chunk decay; its Qt and M slots are not used.  One slice per wave on the
// 128-wide tiles (K = V = 128, or 64 with V = 64 columns).
template <int NW, int VD>
__global__ __launch_bounds__(64 * (NW + 1), NW > 4 ? 1 : 2) void fscan_kernel(
    const uint16_t *__restrict__ v, const uint8_t *__restrict__ srec,
    const int32_t *__restrict__ cu, int N, int T, int H,
    const void *__restrict__ init, int init_fp32, uint16_t *__restrict__ s0, uint16_t *__restrict__ xws)
{
    constexpr int CW = NW * 16;
    constexpr int V = VD;
    constexpr int NT = HD / 16, NKB = HD / 32;
    typedef StatesRec R;
    constexpr int RKB = R::BYTES / 1024;
    constexpr int NSPLIT = V / CW;
    static_assert(NSPLIT * CW == V, "column parts cover the head");
    constexpr int V_KB = CS * CW * 2 / 1024;
    constexpr int UNITS = RKB + V_KB;
    constexpr int VROW_LANES = CW * 2 / 16;
    constexpr int DEPTH = 4;                       // (DEPTH - 1) x 19 DMAs within vmcnt
    __shared__ ScanSlot<CW, R::BYTES> ring[DEPTH];
    static_assert((DEPTH - 1) * UNITS <= 63, "vmcnt holds at most 63");

    const int b = blockIdx.x;
    const int u = 8 * (b / (8 * NSPLIT)) + (b & 7);
    const int part = (b >> 3) % NSPLIT;
    if (u >= N * H) return;                           // block-uniform
    const int n = u / H, h = u % H;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int grp = l >> 4, cg = l & 15;
    const bool dma_wave = w == NW;
    const int wcol0 = (dma_wave ? 0 : w) * 16;
    const int col0 = part * CW;
    const int p16 = (col0 + wcol0) >> 4;

    int64_t start, end;
    seq_range(cu, n, T, start, end);
    const int64_t L = end - start;
    const int nch = (int)((L + CS - 1) / CS);
    const int64_t slot0 = seq_slot0(cu, n, T);
    const size_t row_bytes = (size_t)H * V * 2;

    f32x4_t S[NT];
    if (!dma_wave) {
        const size_t slab = (size_t)V * V * (init_fp32 ? 4 : 2);
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc((const uint8_t *)init + (init ? ((size_t)n * H + h) * slab : 0), init ? (uint32_t)slab : 0u);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = state_chan(t, 4 * grp + j);
                const int idx = row * V + col0 + wcol0 + cg;
                float x = 0.f;
                if (row < V)
                    x = init_fp32 ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, idx * 4, 0, 0))
                                  : bf16f(__builtin_amdgcn_raw_buffer_load_b16(rs, idx * 2, 0, 0));
                S[t][j] = x;
            }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const size_t rec_stride = (size_t)H * R::BYTES;
    const size_t row_stride = (size_t)CS * H * V;
    const uint8_t *rec_base = srec + ((size_t)slot0 * H + h) * R::BYTES;
    const uint16_t *v_base = v + ((size_t)start * H + h) * V + col0;

    auto issue = [&](int c, int slot) {
        const bool live = c < nch;
        const i32x4_t rr =
            rsrc_words(rec_base + (live ? (size_t)c * rec_stride : 0), live ? (uint32_t)R::BYTES : 0u);
        const int64_t rem = L - (int64_t)c * CS;
        const int len = live ? (int)(rem < CS ? rem : CS) : 0;
        const i32x4_t rv =
            rsrc_words(v_base + (live ? (size_t)c * row_stride : 0), (uint32_t)(len * row_bytes));
        ScanSlot<CW, R::BYTES> &sl = ring[slot];
#pragma unroll
        for (int unit = 0; unit < RKB; ++unit) dma16(rr, &sl.rec[unit * 1024], unit * 1024 + l * 16);
#pragma unroll
        for (int vu = 0; vu < V_KB; ++vu) {
            const int vrow0 = vu * (1024 / (2 * CW));
            dma16(rv, &sl.v[vrow0][0], (int)((vrow0 + l / VROW_LANES) * row_bytes) + (l % VROW_LANES) * 16);
        }
    };
    struct Ops {
        u32x4_t kt[NKB], ktl[NKB], wt[NKB], wtl[NKB];
        float gm[2];
        u32x2_t v;
    };
    auto load_ops = [&](int slot, Ops &op) {
        const ScanSlot<CW, R::BYTES> &sl = ring[slot];
        const uint8_t *Rp = sl.rec;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            op.kt[kb] = *(const u32x4_t *)(Rp + R::KTH + (kb * 64 + l) * 16);
            op.ktl[kb] = *(const u32x4_t *)(Rp + R::KTL + (kb * 64 + l) * 16);
            op.wt[kb] = *(const u32x4_t *)(Rp + R::WTH + (kb * 64 + l) * 16);
            op.wtl[kb] = *(const u32x4_t *)(Rp + R::WTL + (kb * 64 + l) * 16);
        }
        const int gch = 32 * (cg >> 2) + 8 * grp + 4 * ((cg >> 1) & 1) + 2 * (cg & 1);
        const u32x2_t g2 = *(const u32x2_t *)(Rp + R::GAM + gch * 4);
        op.gm[0] = __uint_as_float(g2[0]);
        op.gm[1] = __uint_as_float(g2[1]);
        op.v = *(const u32x2_t *)&sl.v[cg][wcol0 + 4 * grp];
    };
    u32x2_t eye;
    {
        const uint32_t one = 0x3f80u;
        const int d = cg - 4 * grp;
        eye[0] = (d == 0 ? one : 0u) | (d == 1 ? one << 16 : 0u);
        eye[1] = (d == 2 ? one : 0u) | (d == 3 ? one << 16 : 0u);
    }
    // Every product is an fp32-accurate sum of three bf16 products of (hi,
    // lo) pairs (the state, X, Kt and Wm), so X and the state match fp32
    // arithmetic closely: the chunk kernel's gradient products take them,
    // and S0 rounded to bf16, as fp32 operands.
    auto hi2 = [](float a, float b) { return pack2(a, b); };
    auto lo2 = [](float a, float b, uint32_t hi) { return pack2(a - bf16lo(hi), b - bf16hi(hi)); };
    auto compute = [&](int c, const Ops &op) {
        const size_t sh = (size_t)(slot0 + c) * H + h;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        u32x4_t Sb[NKB], Sl[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const int t = 2 * kb + (w2 >> 1), j0 = 2 * (w2 & 1);
                const uint32_t hw = hi2(S[t][j0], S[t][j0 + 1]);
                Sb[kb][w2] = hw;
                Sl[kb][w2] = lo2(S[t][j0], S[t][j0 + 1], hw);
            }
        }
        f32x4_t P0 = zero, P1 = zero;
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
            P0 = mfma_k32(op.kt[i], Sb[i], P0);
            P1 = mfma_k32(op.kt[i], Sl[i], P1);
            P1 = mfma_k32(op.ktl[i], Sb[i], P1);
        }
        const f32x4_t vv = mfma_k16(op.v, eye, zero);
        decay_tiles<0, NT>(S, op.gm);
        f32x4_t X;
#pragma unroll
        for (int j = 0; j < 4; ++j) X[j] = vv[j] - (P0[j] + P1[j]);
        const uint32_t xh0 = hi2(X[0], X[1]), xh1 = hi2(X[2], X[3]);
        const u32x2_t Xb = {xh0, xh1}, Xl = {lo2(X[0], X[1], xh0), lo2(X[2], X[3], xh1)};
#pragma unroll
        for (int tp = 0; tp < NKB; ++tp) {
            // tiles 2tp (bf16 0..3) and 2tp+1 (bf16 4..7) of Wm^T, hi and lo parts
            const u32x2_t t0 = {op.wt[tp][0], op.wt[tp][1]}, t1 = {op.wt[tp][2], op.wt[tp][3]};
            const u32x2_t l0 = {op.wtl[tp][0], op.wtl[tp][1]}, l1 = {op.wtl[tp][2], op.wtl[tp][3]};
            S[2 * tp] = mfma_k16(t0, Xb, S[2 * tp]);
            S[2 * tp + 1] = mfma_k16(t1, Xb, S[2 * tp + 1]);
            S[2 * tp] = mfma_k16(t0, Xl, S[2 * tp]);
            S[2 * tp + 1] = mfma_k16(t1, Xl, S[2 * tp + 1]);
            S[2 * tp] = mfma_k16(l0, Xb, S[2 * tp]);
            S[2 * tp + 1] = mfma_k16(l1, Xb, S[2 * tp + 1]);
        }
        // stores (off the chain): X in bf16 through the identity (lane (grp,
        // cg): token cg, columns 4grp .. +3, [16][128] per chunk), S0 in bf16
        // as rows (see rscan_kernel)
        {
            const f32x4_t xt = mfma_k16(Xb, eye, zero);
            const u32x2_t xv = {pack2(xt[0], xt[1]), pack2(xt[2], xt[3])};
            *(u32x2_t *)&xws[sh * CS * HD + cg * HD + col0 + wcol0 + 4 * grp] = xv;
        }
        uint16_t *so = s0 + sh * HD * HD + (size_t)p16 * HD * 16 + 4 * grp;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const u32x2_t a = {Sb[t >> 1][2 * (t & 1)], Sb[t >> 1][2 * (t & 1) + 1]};
            const f32x4_t st = mfma_k16(a, eye, zero);
            const u32x2_t sv = {pack2(st[0], st[1]), pack2(st[2], st[3])};
            *(u32x2_t *)&so[state_chan(t, cg) * 16] = sv;
        }
    };

    if (dma_wave) {
#pragma unroll
        for (int c = 0; c < DEPTH; ++c) issue(c, c);
        wait_vm_barrier<(DEPTH - 1) * UNITS>();
        int slot = 0;
        for (int c = 0; c < nch; ++c) {
            wait_vm_barrier<(DEPTH - 2) * UNITS>();
            issue(c + DEPTH, slot);
            slot = slot == DEPTH - 1 ? 0 : slot + 1;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }
    lds_barrier();
    Ops opA, opB;
    load_ops(0, opA);
    int next = 1;
    auto step = [&](int c, const Ops &cur, Ops &nxt) {
        lds_barrier();
        load_ops(next, nxt);
        compute(c, cur);
        next = next == DEPTH - 1 ? 0 : next + 1;
    };
    for (int c = 0; c < nch; c += 2) {
        step(c, opA, opB);
        if (c + 1 < nch) step(c + 1, opB, opA);
    }
}

int num_cus() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

}  // namespace

hipError_t launch_scan(const uint16_t *v, const uint8_t *ws, const int32_t *cu, int N, int T,
                       int H, int K, int V, float scale, const void *init, int init_fp32,
                       void *fin, int fin_fp32, uint16_t *out, hipStream_t stream, int part_cols)
{
    const int64_t units = (int64_t)N * H;
    if (units <= 0) return hipSuccess;
    // Few (sequence, head) units: split each head's columns over more
    // workgroups (of fewer compute waves) so that more compute units share
    // the scan.  Parts of 32, 64 or 128 columns; V / part workgroups a head.
    const int cus = num_cus();
    // (head dimension 256: parts of 32, 64 or 128 columns, one slice per
    // wave.  The ring of 26 KB records leaves room for one workgroup per
    // compute unit, so past 64 units (on 256 compute units) the parts are
    // 128 columns wide, eight compute waves: two workgroups a head, one
    // round of workgroups up to 128 units.)
    const int cw = V == 2 * HD ? (8 * units <= cus ? 32 : 4 * units <= cus ? 64 : 128)
                 : (V == 128 ? 4 : 2) * units <= cus ? 32 : (V == 128 ? 2 : 1) * units <= cus ? 64 : 128;
    const int part_cw = part_cols ? part_cols : cw > V ? V : cw;
    if ((part_cw != 32 && part_cw != 64 && part_cw != 128) || part_cw > V) return hipErrorInvalidValue;
    const int64_t blocks = 8 * (V / part_cw) * ((units + 7) / 8);
#define KDA_SCAN(CT_, NW_, VD_)                                                               \
    hipLaunchKernelGGL((scan_kernel<CT_, NW_, VD_>), dim3((unsigned)blocks), dim3(64 * (NW_ + 1)), \
                       0, stream, v, ws, cu, N, T, H, scale, init, init_fp32, fin, fin_fp32, out)
    if (V == HD) {
        if (part_cw == 32) KDA_SCAN(1, 2, HD);
        else if (part_cw == 64) KDA_SCAN(1, 4, HD);
        else KDA_SCAN(2, 4, HD);
    } else if (V == 2 * HD) {
        if (part_cw == 32) KDA_SCAN(1, 2, 2 * HD);
        else if (part_cw == 64) KDA_SCAN(1, 4, 2 * HD);
        else KDA_SCAN(1, 8, 2 * HD);
    } else {
        if (part_cw == 32) KDA_SCAN(1, 2, 64);
        else KDA_SCAN(1, 4, 64);
    }
#undef KDA_SCAN
    return hipGetLastError();
}

// Column-part width of the backward's two scans, which run side by side
// (the reverse scan on a second stream): the narrowest of 32, 64 and 128
// columns (V = 64: 32 or 64) at which the workgroups of both fit on the
// compute units at once, one each, else the widest.  A scan workgroup of
// one part cannot share a compute unit with one of the other scan, so a
// width that overfills the chip leaves part of the second scan waiting for
// the first.
int bwd_scan_width(int64_t units, int V) {
    const int64_t cus = num_cus();
    const int64_t u8 = 8 * ((units + 7) / 8);
    for (int cw = 32; cw < V; cw *= 2)
        if (2 * (V / cw) * u8 <= cus) return cw;
    return V;
}

hipError_t launch_bwd_rscan(const uint16_t *dout, const uint8_t *rrec, const int32_t *cu, int N,
                            int T, int H, int V, const float *dfin, float *dinit, uint16_t *dv,
                            uint16_t *ds1, hipStream_t stream)
{
    const int64_t units = (int64_t)N * H;
    if (units <= 0) return hipSuccess;
    const int cw = bwd_scan_width(units, V);
    const int64_t blocks = 8 * (V / cw) * ((units + 7) / 8);
#define KDA_RSCAN(NW_, VD_)                                                                       \
    hipLaunchKernelGGL((rscan_kernel<NW_, VD_>), dim3((unsigned)blocks), dim3(64 * (NW_ + 1)), 0, stream, \
                       dout, rrec, cu, N, T, H, dfin, dinit, dv, ds1)
    if (V == HD) {
        if (cw == 32) KDA_RSCAN(2, HD); else if (cw == 64) KDA_RSCAN(4, HD); else KDA_RSCAN(8, HD);
    } else {
        if (cw == 32) KDA_RSCAN(2, 64); else KDA_RSCAN(4, 64);
    }
#undef KDA_RSCAN
    return hipGetLastError();
}

hipError_t launch_bwd_fscan(const uint16_t *v, const uint8_t *srec, const int32_t *cu, int N, int T,
                            int H, int V, const void *init, int init_fp32, uint16_t *s0, uint16_t *xws,
                            hipStream_t stream)
{
    const int64_t units = (int64_t)N * H;
    if (units <= 0) return hipSuccess;
    const int cw = bwd_scan_width(units, V);
    const int64_t blocks = 8 * (V / cw) * ((units + 7) / 8);
#define KDA_FSCAN(NW_, VD_)                                                                       \
    hipLaunchKernelGGL((fscan_kernel<NW_, VD_>), dim3((unsigned)blocks), dim3(64 * (NW_ + 1)), 0, stream, \
                       v, srec, cu, N, T, H, init, init_fp32, s0, xws)
    if (V == HD) {
        if (cw == 32) KDA_FSCAN(2, HD); else if (cw == 64) KDA_FSCAN(4, HD); else KDA_FSCAN(8, HD);
    } else {
        if (cw == 32) KDA_FSCAN(2, 64); else KDA_FSCAN(4, 64);
    }
#undef KDA_FSCAN
    return hipGetLastError();
}

}  // namespace kda
