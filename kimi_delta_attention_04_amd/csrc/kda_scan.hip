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
#include "kda_scan_dev.h"

namespace kda {

namespace {

// CT 16-column slices per compute wave, NW compute waves (and the DMA wave)
// per workgroup; head dimension K = V = VD (64, 128 or 256), which is also
// the width of the tiles: VD / 16 state row tiles per slice.
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
    constexpr int KTL = VD;                          // key channels of the tiles (64, 128, 256)
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
        // (64-wide tiles: lanes cg < 8 hold the decays of channels 0 .. 63,
        // which are the ones decay_of reads; the others read the record's
        // padding)
#pragma unroll
        for (int p = 0; p < (NKB >= 4 ? NKB / 4 : 1); ++p) {
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

}  // namespace

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

}  // namespace kda
