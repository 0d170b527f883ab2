// 32-token chunks, two kernels: the intra-chunk stage writes one hand-off
// record per (chunk slot, head) (kda_c32_dev.h) and the inter-chunk scan
// consumes them in order.
//
// Scan: a workgroup owns one (sequence, head, column part); each of its NW
// compute waves keeps one 16-column slice of the 128-row fp32 state in MFMA
// accumulators for the whole sequence (columns of the state evolve
// independently).  Per chunk, with the state rows permuted so that the
// accumulators of tile pair (2kb, 2kb+1) rounded to bf16 are the next
// chunk's B operand (state_chan, kda_device.h):
//   P = Kt S (two token row tiles),  X = V - P,
//   O = scale (Qt S + M X) -> bf16,  S = diag(gamma) S + W^T X
// where the two row tiles of X, as the accumulators hold them, are the
// k = 32 B operand of the update and of M X.  The records and the v tiles
// arrive in an LDS ring by buffer-to-LDS DMA from one more wave, DEPTH - 1
// chunks ahead.
#include "kda_c32_dev.h"
#include "kda_launch.h"

namespace kda {

namespace {

template <bool SG>
__global__ __launch_bounds__(64, 2) void intra32_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ g, const uint16_t *__restrict__ beta,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float lb2,
    const int32_t *__restrict__ cu, int N, int T, int H, int K, uint8_t *__restrict__ ws)
{
    __shared__ __attribute__((aligned(16))) Wave32Lds lds;
    __shared__ __attribute__((aligned(16))) Khat32Lds klds;
    __shared__ __attribute__((aligned(16))) float dtb_lds[HD];
    // head fastest; slots last first (see intra_kernel)
    const int64_t slot = (int64_t)(gridDim.x / (unsigned)H) - 1 - blockIdx.x / (unsigned)H;
    const int h = (int)(blockIdx.x % (unsigned)H);
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seq_slot0_32(cu, mid, T) <= slot) lo = mid; else hi = mid - 1;
    }
    const int n = lo;
    int64_t start, end;
    seq_range(cu, n, T, start, end);
    const int64_t t0 = start + (slot - seq_slot0_32(cu, n, T)) * C32;
    if (t0 >= end) return;                             // gap slot, uniform
    const int len = (int)min((int64_t)C32, end - t0);
    uint8_t *rec = ws + ((size_t)slot * H + h) * Rec32::BYTES;

    const float A = expf(A_log[h]);
    stage_dtb<SG, HD>(dtb_lds, dt_bias, h, K);
    wave_lds_sync();
    Intra32Src in;
    intra32_src<SG>(in, q, k, g, beta, t0, len, H, h, K);
    if (len == C32)
        intra32_compute<true, SG>(lds, &klds, in, A, dtb_lds, lb2, len, rec);
    else
        intra32_compute<false, SG>(lds, &klds, in, A, dtb_lds, lb2, len, rec);
}

// s_waitcnt vmcnt(n) followed by a workgroup barrier (waits for this
// wave's LDS traffic too, not for its other global accesses).
template <int NV>
__device__ __forceinline__ void wait_vm_barrier32() {
    static_assert(NV >= 0 && NV <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(NV) : "memory");
}
__device__ __forceinline__ void lds_barrier32() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t rsrc_words32(const void *p, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    i32x4_t r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}
// 16-byte-per-lane buffer-to-LDS DMA (lane l's 16 bytes at `off` land at
// lds + 16 l), from inline assembly so that the compiler's waits do not
// serialise the ring; the waits are explicit (wait_vm_barrier32).
__device__ __forceinline__ void dma16_32(i32x4_t rs, const void *lds, int off) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(off), "s"(rs) : "memory", "m0");
}

template <int CW>
struct alignas(16) Scan32Slot {
    uint8_t rec[Rec32::BYTES];
    uint16_t v[C32][CW];
};

template <int SRC>
__device__ __forceinline__ float row_bcast32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                              0x150 + SRC, 0xf, 0xf, true));
}
// Chunk decay of state row chan(t, 4grp + j): lane 4(t/2) + 2(t%2) + j/2
// of the row holds it in gm[j%2] (see load_ops).
template <int T, int J>
__device__ __forceinline__ float decay32(const float (&gm)[2]) {
    return row_bcast32<4 * (T >> 1) + 2 * (T & 1) + (J >> 1)>(gm[J & 1]);
}
template <int T>
__device__ __forceinline__ void decay_tiles32(f32x4_t (&S)[8], const float (&gm)[2]) {
    if constexpr (T < 8) {
        S[T][0] *= decay32<T, 0>(gm);
        S[T][1] *= decay32<T, 1>(gm);
        S[T][2] *= decay32<T, 2>(gm);
        S[T][3] *= decay32<T, 3>(gm);
        decay_tiles32<T + 1>(S, gm);
    }
}

struct Ops32 {
    u32x4_t kt[4][2], qt[4][2], wt[8], m[2];
    float gm[2];
    u32x2_t v[2];
};

constexpr int ring_depth32(int units) { return 63 / units + 2 > 4 ? 4 : 63 / units + 2; }

// NW compute waves of one 16-column slice each, plus the DMA wave; VD = 128,
// or 64 on the 128-wide tiles (state rows and columns from 64 on zero).
template <int NW, int VD>
__global__ __launch_bounds__(64 * (NW + 1), 1) void scan32_kernel(
    const uint16_t *__restrict__ v, const uint8_t *__restrict__ ws,
    const int32_t *__restrict__ cu, int N, int T, int H, float scale,
    const void *__restrict__ init, int init_fp32,
    void *__restrict__ fin, int fin_fp32, uint16_t *__restrict__ out)
{
    constexpr int CW = NW * 16;
    constexpr int K = VD, V = VD;
    constexpr int NSPLIT = V / CW;
    static_assert(NSPLIT * CW == V, "column parts cover the head");
    constexpr int RKB = Rec32::BYTES / 1024;
    constexpr int V_KB = C32 * CW * 2 / 1024;
    constexpr int UNITS = RKB + V_KB;
    constexpr int VROW_LANES = CW * 2 / 16;
    constexpr int DEPTH = ring_depth32(UNITS);
    static_assert((DEPTH - 2) * UNITS <= 63 && DEPTH >= 3, "vmcnt holds at most 63");
    __shared__ Scan32Slot<CW> ring[DEPTH];

    const int b = blockIdx.x;
    const int u = 8 * (b / (8 * NSPLIT)) + (b & 7);
    const int part = (b >> 3) % NSPLIT;
    if (u >= N * H) return;
    const int n = u / H, h = u % H;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int grp = l >> 4, cg = l & 15;
    const bool dma_wave = w == NW;
    const int wcol0 = (dma_wave ? 0 : w) * 16;
    const int col0 = part * CW;

    int64_t start, end;
    seq_range(cu, n, T, start, end);
    const int64_t L = end - start;
    const int nch = __builtin_amdgcn_readfirstlane((int)((L + C32 - 1) / C32));
    const int64_t slot0 = seq_slot0_32(cu, n, T);
    const size_t row_bytes = (size_t)H * V * 2;

    f32x4_t S[8];
    if (!dma_wave) {
        const size_t slab = (size_t)K * V * (init_fp32 ? 4 : 2);
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc((const uint8_t *)init + (init ? ((size_t)n * H + h) * slab : 0),
                      init ? (uint32_t)slab : 0u);
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int idx = state_chan(t, 4 * grp + j) * V + col0 + wcol0 + cg;
                S[t][j] = init_fp32
                    ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, idx * 4, 0, 0))
                    : bf16f(__builtin_amdgcn_raw_buffer_load_b16(rs, idx * 2, 0, 0));
            }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const size_t rec_stride = (size_t)H * Rec32::BYTES;
    const size_t row_stride = (size_t)C32 * H * V;
    const uint8_t *rec_base = ws + ((size_t)slot0 * H + h) * Rec32::BYTES;
    const uint16_t *v_base = v + ((size_t)start * H + h) * V + col0;
    uint16_t *out_base = out + ((size_t)start * H + h) * V + col0;

    auto issue = [&](int c, int slot) {
        const bool live = c < nch;
        const i32x4_t rr = rsrc_words32(rec_base + (live ? (size_t)c * rec_stride : 0),
                                        live ? (uint32_t)Rec32::BYTES : 0u);
        const int64_t rem = L - (int64_t)c * C32;
        const int len = live ? (int)(rem < C32 ? rem : C32) : 0;
        const i32x4_t rv = rsrc_words32(v_base + (live ? (size_t)c * row_stride : 0),
                                        (uint32_t)(len * row_bytes));
        Scan32Slot<CW> &sl = ring[slot];
#pragma unroll
        for (int unit = 0; unit < RKB; ++unit) dma16_32(rr, &sl.rec[unit * 1024], unit * 1024 + l * 16);
#pragma unroll
        for (int vu = 0; vu < V_KB; ++vu) {
            const int vrow0 = vu * (1024 / (2 * CW));
            dma16_32(rv, &sl.v[vrow0][0], (int)((vrow0 + l / VROW_LANES) * row_bytes) + (l % VROW_LANES) * 16);
        }
    };

    auto load_ops = [&](int slot, Ops32 &op) {
        const Scan32Slot<CW> &sl = ring[slot];
        const uint8_t *Rp = sl.rec;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                op.kt[kb][rt] = *(const u32x4_t *)(Rp + Rec32::KT + ((kb * 2 + rt) * 64 + l) * 16);
                op.qt[kb][rt] = *(const u32x4_t *)(Rp + Rec32::QT + ((kb * 2 + rt) * 64 + l) * 16);
            }
#pragma unroll
        for (int t = 0; t < 8; ++t) op.wt[t] = *(const u32x4_t *)(Rp + Rec32::WT + (t * 64 + l) * 16);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) op.m[rt] = *(const u32x4_t *)(Rp + Rec32::M + (rt * 64 + l) * 16);
        const int gch = 32 * (cg >> 2) + 8 * grp + 4 * ((cg >> 1) & 1) + 2 * (cg & 1);
        const u32x2_t g2 = *(const u32x2_t *)(Rp + Rec32::GAM + gch * 4);
        op.gm[0] = __uint_as_float(g2[0]);
        op.gm[1] = __uint_as_float(g2[1]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) op.v[rt] = *(const u32x2_t *)&sl.v[16 * rt + cg][wcol0 + 4 * grp];
    };

    u32x2_t eye;
    {
        const uint32_t one = 0x3f80u;
        const int d = cg - 4 * grp;
        eye[0] = (d == 0 ? one : 0u) | (d == 1 ? one << 16 : 0u);
        eye[1] = (d == 2 ? one : 0u) | (d == 3 ? one << 16 : 0u);
    }
    auto compute = [&](int c, const Ops32 &op) {
        const int64_t rem = L - (int64_t)c * C32;
        const int len = (int)(rem < C32 ? rem : C32);
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(out_base + (size_t)c * row_stride, (uint32_t)((len - 1) * row_bytes + CW * 2));
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        u32x4_t Sb[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            Sb[kb][0] = pack2(S[2 * kb][0], S[2 * kb][1]);
            Sb[kb][1] = pack2(S[2 * kb][2], S[2 * kb][3]);
            Sb[kb][2] = pack2(S[2 * kb + 1][0], S[2 * kb + 1][1]);
            Sb[kb][3] = pack2(S[2 * kb + 1][2], S[2 * kb + 1][3]);
        }
        f32x4_t P[2] = {zero, zero}, Qs[2] = {zero, zero}, vv[2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) P[rt] = mfma_k32(op.kt[kb][rt], Sb[kb], P[rt]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) vv[rt] = mfma_k16(op.v[rt], eye, zero);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) Qs[rt] = mfma_k32(op.qt[kb][rt], Sb[kb], Qs[rt]);
        decay_tiles32<0>(S, op.gm);
        u32x4_t Xb;
        Xb[0] = pack2(vv[0][0] - P[0][0], vv[0][1] - P[0][1]);
        Xb[1] = pack2(vv[0][2] - P[0][2], vv[0][3] - P[0][3]);
        Xb[2] = pack2(vv[1][0] - P[1][0], vv[1][1] - P[1][1]);
        Xb[3] = pack2(vv[1][2] - P[1][2], vv[1][3] - P[1][3]);
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = mfma_k32(op.wt[t], Xb, S[t]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const f32x4_t MX = mfma_k32(op.m[rt], Xb, zero);
            const u32x2_t oa = {pack2(scale * (Qs[rt][0] + MX[0]), scale * (Qs[rt][1] + MX[1])),
                                pack2(scale * (Qs[rt][2] + MX[2]), scale * (Qs[rt][3] + MX[3]))};
            const f32x4_t ot = mfma_k16(oa, eye, zero);
            const u32x2_t os = {pack2(ot[0], ot[1]), pack2(ot[2], ot[3])};
            __builtin_amdgcn_raw_buffer_store_b64(
                os, ro, (int)((16 * rt + cg) * row_bytes) + (wcol0 + 4 * grp) * 2, 0, 0);
        }
    };

    if (dma_wave) {
#pragma unroll
        for (int c = 0; c < DEPTH - 1; ++c) issue(c, c);
        int slot = DEPTH - 1;                        // ring slot of chunk c-1
        for (int c = 0; c < nch; ++c) {
            wait_vm_barrier32<(DEPTH - 2) * UNITS>();   // chunk c landed; slot of c-1 free
            issue(c - 1 + DEPTH, slot);
            slot = slot == DEPTH - 1 ? 0 : slot + 1;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }
    Ops32 op;
    int cur = 0;
    for (int c = 0; c < nch; ++c) {
        lds_barrier32();                             // own reads of c-1 done; chunk c landed
        load_ops(cur, op);
        compute(c, op);
        cur = cur == DEPTH - 1 ? 0 : cur + 1;
    }

    if (fin) {
        const size_t slab = (size_t)K * V * (fin_fp32 ? 4 : 2);
        const __amdgpu_buffer_rsrc_t rf =
            make_rsrc((uint8_t *)fin + ((size_t)n * H + h) * slab, (uint32_t)slab);
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int idx = state_chan(t, 4 * grp + j) * V + col0 + wcol0 + cg;
                if (fin_fp32)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[t][j]), rf, idx * 4, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16(tobf16(S[t][j]), rf, idx * 2, 0, 0);
            }
    }
}

int cu_count32() {
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

int64_t c32_num_slots(int64_t tokens, int N) { return tokens / C32 + N; }

hipError_t launch_intra32(const uint16_t *q, const uint16_t *k, const uint16_t *g,
                          const uint16_t *beta, const float *A_log, const float *dt_bias,
                          float lower_bound, const int32_t *cu, int N, int T, int H, int K,
                          int64_t num_slots, uint8_t *ws, hipStream_t stream, bool scalar_gate)
{
    if (num_slots <= 0) return hipSuccess;
    dim3 grid((unsigned)(num_slots * H));
    const float lb2 = lower_bound * LOG2E;
    if (scalar_gate)
        hipLaunchKernelGGL((intra32_kernel<true>), grid, dim3(64), 0, stream, q, k, g, beta, A_log,
                           dt_bias, lb2, cu, N, T, H, K, ws);
    else
        hipLaunchKernelGGL((intra32_kernel<false>), grid, dim3(64), 0, stream, q, k, g, beta, A_log,
                           dt_bias, lb2, cu, N, T, H, K, ws);
    return hipGetLastError();
}

hipError_t launch_scan32(const uint16_t *v, const uint8_t *ws, const int32_t *cu, int N, int T,
                         int H, int K, int V, float scale, const void *init, int init_fp32,
                         void *fin, int fin_fp32, uint16_t *out, hipStream_t stream, int part_cols)
{
    const int64_t units = (int64_t)N * H;
    if (units <= 0) return hipSuccess;
    const int cus = cu_count32();
    // columns per workgroup: 32 while four parts a head still leave compute
    // units free, then 64, then the whole head (unless the caller fixes it)
    int cw = (V / 32) * units <= cus ? 32 : (V / 64) * units <= cus ? 64 : 128;
    if (part_cols) cw = part_cols;
    if (cw > V) cw = V;
    if (cw != 32 && cw != 64 && cw != 128) return hipErrorInvalidValue;
    const int64_t blocks = 8 * (V / cw) * ((units + 7) / 8);
#define KDA_SCAN32(NW_, VD_)                                                                     \
    hipLaunchKernelGGL((scan32_kernel<NW_, VD_>), dim3((unsigned)blocks), dim3(64 * (NW_ + 1)), 0, \
                       stream, v, ws, cu, N, T, H, scale, init, init_fp32, fin, fin_fp32, out)
    if (V == HD) {
        if (cw == 32) KDA_SCAN32(2, HD);
        else if (cw == 64) KDA_SCAN32(4, HD);
        else KDA_SCAN32(8, HD);
    } else {
        if (cw == 32) KDA_SCAN32(2, 64);
        else KDA_SCAN32(4, 64);
    }
#undef KDA_SCAN32
    return hipGetLastError();
}

}  // namespace kda
