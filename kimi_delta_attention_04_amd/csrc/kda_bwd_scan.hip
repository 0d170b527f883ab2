// The backward's two scans on the forward scan's structure (kda_scan.hip):
// a workgroup owns one (sequence, head, column part), each of its NW compute
// waves one 16-column slice of the 128-row state in MFMA accumulators, and
// one more wave fills an LDS ring with each chunk's record and token tile by
// DMA (kda_scan_dev.h).  The states scan runs the chunk recurrence forward
// from the initial state and stores the start state S0 of a sequence's even
// chunks and every chunk's X; the reverse scan runs the state gradient
// backward from d_final_state and stores dS1 of the odd chunks and of the
// last one, and dv (= dX).  The chunk kernel rebuilds the other half's
// products from the neighbouring chunk.  They are independent (both read
// only the prep kernel's records and the token inputs), and the backward
// launches them side by side on two streams.
#include "kda_device.h"
#include "kda_bwd_dev.h"
#include "kda_launch.h"
#include "kda_scan_dev.h"

namespace kda {

namespace {

// Ring slots of the backward's scans: as many as the DMA wave's vmcnt (at
// most 63 one-kilobyte DMAs outstanding: DEPTH-1 chunks of UNITS each, or
// DEPTH-2 when the DMA wave refills a slot one chunk late) allows, at most 8.  The scans store a state every other
// chunk, and their record and token-tile reads queue behind those stores, so
// they run with as many chunks in flight as fit (at K = V = 64 the two scans
// take 0.41 ms with 8 slots against 0.57 ms with 4 or 5; at 128 the depth
// changes nothing measurable).
template <int UNITS, bool LAG>
constexpr int bwd_ring_depth() {
    return 63 / UNITS + (LAG ? 2 : 1) > 8 ? 8 : 63 / UNITS + (LAG ? 2 : 1);
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
// Stored for the chunk kernel: dS1 rounded to bf16 (odd chunks of the
// sequence and the last one), as rows of each 16-column part ([part][row]
// [16 columns]), and dV = dX in bf16.
// One slice per wave on tiles as wide as the head (K = V = VD, 64 or 128).
template <int NW, int VD>
__global__ __launch_bounds__(64 * (NW + 1), NW > 4 ? 1 : 2) void rscan_kernel(
    const uint16_t *__restrict__ dout, const uint8_t *__restrict__ rrec,
    const int32_t *__restrict__ cu, int N, int T, int H,
    const float *__restrict__ dfin, float *__restrict__ dinit, uint16_t *__restrict__ dv,
    uint16_t *__restrict__ ds1)
{
    constexpr int CW = NW * 16;
    constexpr int V = VD;
    constexpr int NT = VD / 16, NKB = VD / 32;
    typedef RecLayout<VD> R;
    constexpr int RKB = R::BYTES / 1024;
    constexpr int NSPLIT = V / CW;
    static_assert(NSPLIT * CW == V, "column parts cover the head");
    constexpr int V_KB = CS * CW * 2 / 1024;
    constexpr int UNITS = RKB + V_KB;
    constexpr int VROW_LANES = CW * 2 / 16;
    // LAG (eight compute waves, which must fit 168 registers: three waves
    // share a SIMD): the compute waves read a chunk's state-update operands
    // (scale Qt, -Kt) at the top of its own iteration instead of one chunk
    // ahead, and the DMA wave refills a slot one chunk later (chunk c-1's
    // slot in iteration c).
    // ONESET (256-wide tiles): one operand set in registers, all of chunk
    // c's operands read at the top of iteration c, and the DMA wave refilling
    // chunk c-1's slot, as the forward scan does at that width.
    constexpr bool ONESET = VD > HD;
    constexpr bool LAG = !ONESET && NW > 4;
    constexpr int DEPTH = bwd_ring_depth<UNITS, LAG || ONESET>();
    __shared__ ScanSlot<CW, R::BYTES> ring[DEPTH];
    static_assert((DEPTH - (LAG || ONESET ? 2 : 1)) * UNITS <= 63, "vmcnt holds at most 63");

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
                const int idx = state_chan(t, 4 * grp + j) * V + col0 + wcol0 + cg;
                S[t][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, idx * 4, 0, 0));
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
    // the state-update operands (scale Qt and -Kt in the W^T layout)
    auto load_update = [&](int slot, ChunkOps<1, NKB> &op) {
        const uint8_t *Rp = ring[slot].rec;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            op.qt[kb] = *(const u32x4_t *)(Rp + R::QT + (kb * 64 + l) * 16);
            op.wt[kb] = *(const u32x4_t *)(Rp + R::WT + (kb * 64 + l) * 16);
        }
    };
    // the chunk's other operands, and (not LAG) the update operands
    auto load_ops = [&](int slot, ChunkOps<1, NKB> &op) {
        const ScanSlot<CW, R::BYTES> &sl = ring[slot];
        const uint8_t *Rp = sl.rec;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) op.kt[kb] = *(const u32x4_t *)(Rp + R::KTO + (kb * 64 + l) * 16);
        if constexpr (!LAG) load_update(slot, op);
        op.m = *(const u32x2_t *)(Rp + R::M + l * 8);
        const int gch = 32 * (cg >> 2) + 8 * grp + 4 * ((cg >> 1) & 1) + 2 * (cg & 1);
#pragma unroll
        for (int p = 0; p < (NKB >= 4 ? NKB / 4 : 1); ++p) {
            const u32x2_t g2 = *(const u32x2_t *)(Rp + R::GAM + (128 * p + gch) * 4);
            op.gm[2 * p] = __uint_as_float(g2[0]);
            op.gm[2 * p + 1] = __uint_as_float(g2[1]);
        }
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
        // dS1 of the odd chunks and of the last one only (the chunk kernel
        // rebuilds an even chunk's products from the chunk after)
        uint16_t *so = ds1 + sh * V * V + (size_t)p16 * V * 16 + 4 * grp;
        if ((ci & 1) == 1 || ci == nch - 1)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const u32x2_t a = {Sb[t >> 1][2 * (t & 1)], Sb[t >> 1][2 * (t & 1) + 1]};
            const f32x4_t st = mfma_k16(a, eye, zero);
            const u32x2_t sv = {pack2(st[0], st[1]), pack2(st[2], st[3])};
            *(u32x2_t *)&so[state_chan(t, cg) * 16] = sv;
        }
    };

    // Ring protocols (chunk c in ring slot c % DEPTH).  Two operand sets
    // (the forward scan's): the compute waves read chunk c+1's operands in
    // iteration c and the DMA wave refills chunk c's slot in iteration c.
    // LAG: as that, but the update operands of chunk c are read in iteration
    // c, so the DMA wave refills chunk c-1's slot; DEPTH-1 chunks go out
    // before the first iteration, and at the top of iteration c chunk c+1
    // has landed when the DMAs issued after its own number (DEPTH-3) UNITS.
    // ONESET: all of chunk c's operands are read in iteration c, the DMA
    // wave refills chunk c-1's slot, and at the top of iteration c chunk c
    // has landed when (DEPTH-2) UNITS remain.
    if (dma_wave) {
        if constexpr (ONESET) {
#pragma unroll
            for (int c = 0; c < DEPTH - 1; ++c) issue(c, c);
            int slot = DEPTH - 1;                     // ring slot of chunk c-1
            for (int c = 0; c < nch; ++c) {
                wait_vm_barrier<(DEPTH - 2) * UNITS>();  // chunk c landed; slot of c-1 free
                issue(c - 1 + DEPTH, slot);
                slot = slot == DEPTH - 1 ? 0 : slot + 1;
            }
        } else if constexpr (LAG) {
#pragma unroll
            for (int c = 0; c < DEPTH - 1; ++c) issue(c, c);
            wait_vm_barrier<(DEPTH - 2) * UNITS>();   // chunk 0 landed
            int slot = DEPTH - 1;                     // ring slot of chunk c-1
            for (int c = 0; c < nch; ++c) {
                wait_vm_barrier<(DEPTH - 3) * UNITS>();  // chunk c+1 landed; slot of c-1 free
                issue(c + DEPTH - 1, slot);
                slot = slot == DEPTH - 1 ? 0 : slot + 1;
            }
        } else {
#pragma unroll
            for (int c = 0; c < DEPTH; ++c) issue(c, c);
            wait_vm_barrier<(DEPTH - 1) * UNITS>();
            int slot = 0;
            for (int c = 0; c < nch; ++c) {
                wait_vm_barrier<(DEPTH - 2) * UNITS>();
                issue(c + DEPTH, slot);
                slot = slot == DEPTH - 1 ? 0 : slot + 1;
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }
    if constexpr (ONESET) {
        ChunkOps<1, NKB> op;
        int cur = 0;                                  // ring slot of chunk c
        for (int c = 0; c < nch; ++c) {
            lds_barrier();                            // own reads of chunk c-1 done; chunk c landed
            load_ops(cur, op);
            compute(c, op);
            cur = cur == DEPTH - 1 ? 0 : cur + 1;
        }
    } else {
        lds_barrier();
        ChunkOps<1, NKB> opA, opB;
        load_ops(0, opA);
        int cur = 0;                                  // ring slot of chunk c
        auto step = [&](int c, ChunkOps<1, NKB> &now, ChunkOps<1, NKB> &nxt) {
            lds_barrier();                            // own reads of chunk c-1 done; chunk c+1 landed
            const int next = cur == DEPTH - 1 ? 0 : cur + 1;
            load_ops(next, nxt);
            if constexpr (LAG) load_update(cur, now);
            compute(c, now);
            cur = next;
        };
        for (int c = 0; c < nch; c += 2) {
            step(c, opA, opB);
            if (c + 1 < nch) step(c + 1, opB, opA);
        }
    }
    if (dinit) {
        const size_t base = ((size_t)n * H + h) * V * V;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dinit[base + (size_t)state_chan(t, 4 * grp + j) * V + col0 + wcol0 + cg] = S[t][j];
            }
    }
}

// Forward scan of the backward pass: the state S of one (sequence, head)
// from the initial state through every chunk (X = V - Kt S0,
// S1 = diag(gamma) S0 + Wm^T X, with the state and X as (hi, lo) bf16
// operands), without the output, storing
// for the chunk kernel the start state S0 rounded to bf16 of the sequence's
// even chunks (rows of each 16-column part, [part][VD rows][16 columns])
// and X in bf16 ([16][V]) of every chunk.  The record of each chunk
// (StatesRecT<VD>, written by the backward's prep kernel) holds Kt and Wm in
// the forward record's Kt and W^T layouts and the chunk decay.  One slice
// per wave on tiles as wide as the head (K = V = VD, 64 or 128).
template <int NW, int VD>
__global__ __launch_bounds__(64 * (NW + 1), NW > 4 ? 1 : 2) void fscan_kernel(
    const uint16_t *__restrict__ v, const uint8_t *__restrict__ srec,
    const int32_t *__restrict__ cu, int N, int T, int H,
    const void *__restrict__ init, int init_fp32, uint16_t *__restrict__ s0, uint16_t *__restrict__ xws)
{
    constexpr int CW = NW * 16;
    constexpr int V = VD;
    constexpr int NT = VD / 16, NKB = VD / 32;
    typedef StatesRecT<VD> R;
    constexpr int RKB = R::BYTES / 1024;
    constexpr int NSPLIT = V / CW;
    static_assert(NSPLIT * CW == V, "column parts cover the head");
    constexpr int V_KB = CS * CW * 2 / 1024;
    constexpr int UNITS = RKB + V_KB;
    constexpr int VROW_LANES = CW * 2 / 16;
    constexpr bool ONESET = VD > HD;                // as in rscan_kernel
    constexpr int DEPTH = bwd_ring_depth<UNITS, ONESET>();
    __shared__ ScanSlot<CW, R::BYTES> ring[DEPTH];
    static_assert((DEPTH - (ONESET ? 2 : 1)) * UNITS <= 63, "vmcnt holds at most 63");

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
                const int idx = state_chan(t, 4 * grp + j) * V + col0 + wcol0 + cg;
                S[t][j] = init_fp32 ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, idx * 4, 0, 0))
                                    : bf16f(__builtin_amdgcn_raw_buffer_load_b16(rs, idx * 2, 0, 0));
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
        u32x4_t kt[NKB], wt[NKB];
        float gm[NKB >= 4 ? NKB / 2 : 2];
        u32x2_t v;
    };
    auto load_ops = [&](int slot, Ops &op) {
        const ScanSlot<CW, R::BYTES> &sl = ring[slot];
        const uint8_t *Rp = sl.rec;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            op.kt[kb] = *(const u32x4_t *)(Rp + R::KTH + (kb * 64 + l) * 16);
            op.wt[kb] = *(const u32x4_t *)(Rp + R::WTH + (kb * 64 + l) * 16);
        }
        const int gch = 32 * (cg >> 2) + 8 * grp + 4 * ((cg >> 1) & 1) + 2 * (cg & 1);
#pragma unroll
        for (int p = 0; p < (NKB >= 4 ? NKB / 4 : 1); ++p) {
            const u32x2_t g2 = *(const u32x2_t *)(Rp + R::GAM + (128 * p + gch) * 4);
            op.gm[2 * p] = __uint_as_float(g2[0]);
            op.gm[2 * p + 1] = __uint_as_float(g2[1]);
        }
        op.v = *(const u32x2_t *)&sl.v[cg][wcol0 + 4 * grp];
    };
    u32x2_t eye;
    {
        const uint32_t one = 0x3f80u;
        const int d = cg - 4 * grp;
        eye[0] = (d == 0 ? one : 0u) | (d == 1 ? one << 16 : 0u);
        eye[1] = (d == 2 ? one : 0u) | (d == 3 ? one << 16 : 0u);
    }
    // The state and X enter their products as (hi, lo) bf16 pairs, Kt and
    // Wm as bf16 (two products each): the recurrence keeps the state's fp32
    // accumulation, and the chunk kernel takes S0 and X rounded to bf16.
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
            // tiles 2tp (bf16 0..3) and 2tp+1 (bf16 4..7) of Wm^T
            const u32x2_t t0 = {op.wt[tp][0], op.wt[tp][1]}, t1 = {op.wt[tp][2], op.wt[tp][3]};
            S[2 * tp] = mfma_k16(t0, Xb, S[2 * tp]);
            S[2 * tp + 1] = mfma_k16(t1, Xb, S[2 * tp + 1]);
            S[2 * tp] = mfma_k16(t0, Xl, S[2 * tp]);
            S[2 * tp + 1] = mfma_k16(t1, Xl, S[2 * tp + 1]);
        }
        // stores (off the chain): X in bf16 through the identity (lane (grp,
        // cg): token cg, columns 4grp .. +3, [16][V] per chunk), S0 in bf16
        // as rows (see rscan_kernel)
        {
            const f32x4_t xt = mfma_k16(Xb, eye, zero);
            const u32x2_t xv = {pack2(xt[0], xt[1]), pack2(xt[2], xt[3])};
            *(u32x2_t *)&xws[sh * CS * V + cg * V + col0 + wcol0 + 4 * grp] = xv;
        }
        // S0 of the even chunks only (the chunk kernel rebuilds an odd
        // chunk's products from the chunk before)
        uint16_t *so = s0 + sh * V * V + (size_t)p16 * V * 16 + 4 * grp;
        if ((c & 1) == 0)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const u32x2_t a = {Sb[t >> 1][2 * (t & 1)], Sb[t >> 1][2 * (t & 1) + 1]};
            const f32x4_t st = mfma_k16(a, eye, zero);
            const u32x2_t sv = {pack2(st[0], st[1]), pack2(st[2], st[3])};
            *(u32x2_t *)&so[state_chan(t, cg) * 16] = sv;
        }
    };

    if (dma_wave) {
        if constexpr (ONESET) {
#pragma unroll
            for (int c = 0; c < DEPTH - 1; ++c) issue(c, c);
            int slot = DEPTH - 1;                     // ring slot of chunk c-1
            for (int c = 0; c < nch; ++c) {
                wait_vm_barrier<(DEPTH - 2) * UNITS>();  // chunk c landed; slot of c-1 free
                issue(c - 1 + DEPTH, slot);
                slot = slot == DEPTH - 1 ? 0 : slot + 1;
            }
        } else {
#pragma unroll
            for (int c = 0; c < DEPTH; ++c) issue(c, c);
            wait_vm_barrier<(DEPTH - 1) * UNITS>();
            int slot = 0;
            for (int c = 0; c < nch; ++c) {
                wait_vm_barrier<(DEPTH - 2) * UNITS>();
                issue(c + DEPTH, slot);
                slot = slot == DEPTH - 1 ? 0 : slot + 1;
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }
    if constexpr (ONESET) {
        Ops op;
        int cur = 0;                                  // ring slot of chunk c
        for (int c = 0; c < nch; ++c) {
            lds_barrier();                            // own reads of chunk c-1 done; chunk c landed
            load_ops(cur, op);
            compute(c, op);
            cur = cur == DEPTH - 1 ? 0 : cur + 1;
        }
    } else {
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
}

}  // namespace

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
    // 256-wide tiles: parts of at most 64 columns.  128-column parts (eight
    // compute waves of 152-161 registers) measure the same at T = 8192,
    // H = 96 (6.60 ms per backward step): there the two scans' workgroups
    // outnumber the compute units at either width.
    const int widest = V > HD ? 64 : V;
    for (int cw = 32; cw < widest; cw *= 2)
        if (2 * (V / cw) * u8 <= cus) return cw;
    return widest;
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
    } else if (V == 2 * HD) {
        if (cw == 32) KDA_RSCAN(2, 2 * HD); else KDA_RSCAN(4, 2 * HD);
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
    } else if (V == 2 * HD) {
        if (cw == 32) KDA_FSCAN(2, 2 * HD); else KDA_FSCAN(4, 2 * HD);
    } else {
        if (cw == 32) KDA_FSCAN(2, 64); else KDA_FSCAN(4, 64);
    }
#undef KDA_FSCAN
    return hipGetLastError();
}

}  // namespace kda
