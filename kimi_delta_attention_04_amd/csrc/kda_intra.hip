// Intra-chunk stage: token-parallel over (chunk slot, head), one wave (a
// workgroup of its own) per pair, writing the hand-off record the scan
// consumes into global memory.  The arithmetic is intra_compute
// (kda_intra_dev.h).
#include "kda_intra_dev.h"
#include "kda_launch.h"

namespace kda {

namespace {

// One wave per (chunk slot, head), a workgroup of its own.  SG: scalar
// (per-head) gate, g [B*T, H] and dt_bias [H].  KD: head dimension (64,
// 128 or 256), the width of the tiles and of the record.
template <bool SG, int KD>
__global__ __launch_bounds__(64, 2) void intra_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ g, const uint16_t *__restrict__ beta,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float lb2,
    const int32_t *__restrict__ cu, int N, int T, int H, uint8_t *__restrict__ ws)
{
    constexpr int K = KD;
    constexpr int KT = KD;                        // channels of the tiles
    __shared__ __attribute__((aligned(16))) WaveLdsT<KT> lds;
    // Head fastest: the workgroups running together read neighbouring pieces
    // of the same token rows and write neighbouring records.  The records
    // are stored non-temporally: written the normal way they stay dirty in
    // the memory-side cache and are written back while the scan runs
    // (measured at T = 8192, H = 96: intra 234 -> 243 us, scan 307 -> 292 us,
    // the two together 7 us faster).  Slots run last first, which helped
    // when the records went through that cache (the scan's first records
    // were the freshest); with non-temporal stores either order measures
    // the same.
    const int64_t slot = (int64_t)(gridDim.x / (unsigned)H) - 1 - blockIdx.x / (unsigned)H;
    const int h = (int)(blockIdx.x % (unsigned)H);

    // Which sequence owns this slot: largest n with slot0(n) <= slot.
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (seq_slot0(cu, mid, T) <= slot) lo = mid; else hi = mid - 1;
    }
    const int n = lo;
    int64_t start, end;
    seq_range(cu, n, T, start, end);
    const int64_t t0 = start + (slot - seq_slot0(cu, n, T)) * CS;
    if (t0 >= end) return;                         // gap slot, wave-uniform
    const int len = (int)min((int64_t)CS, end - t0);
    uint8_t *rec = ws + ((size_t)slot * H + h) * RecLayout<KT>::BYTES;

    const float A = expf(A_log[h]);
    __shared__ float dtb_lds[KT];
    stage_dtb<SG, KT>(dtb_lds, dt_bias, h, K);
    wave_lds_sync();

    IntraInT<KT / 32> in;
    intra_load<SG, KT>(in, q, k, g, beta, t0, len, H, h, K);
    if (len == CS)
        intra_compute<true, SG, KT>(lds, in, A, dtb_lds, lb2, len, rec);
    else
        intra_compute<false, SG, KT>(lds, in, A, dtb_lds, lb2, len, rec);
}

// The gate stage alone: one wave per (chunk slot, head) as in intra_kernel,
// through the same gate code (gate_cumsum, beta_sigmoid).  For every token
// of the chunk it writes the in-chunk inclusive cumulative base-2 log-decay
// G [token, head, channel] and beta [token, head], both fp32.
template <int KD>
__global__ __launch_bounds__(64) void gate_kernel(
    const uint16_t *__restrict__ g, const uint16_t *__restrict__ beta,
    const float *__restrict__ A_log, const float *__restrict__ dt_bias, float lb2,
    const int32_t *__restrict__ cu, int N, int T, int H, float *__restrict__ G_out,
    float *__restrict__ beta_out)
{
    constexpr int NKB = KD / 32;
    const int64_t slot = blockIdx.x / (unsigned)H;
    const int h = (int)(blockIdx.x % (unsigned)H);
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (seq_slot0(cu, mid, T) <= slot) lo = mid; else hi = mid - 1;
    }
    int64_t start, end;
    seq_range(cu, lo, T, start, end);
    const int64_t t0 = start + (slot - seq_slot0(cu, lo, T)) * CS;
    if (t0 >= end) return;                         // gap slot, wave-uniform
    const int len = (int)min((int64_t)CS, end - t0);

    const int l = threadIdx.x, tok = l & 15, grp = l >> 4;
    const bool live = tok < len;
    const float A = expf(A_log[h]);
    __shared__ float dtb_lds[KD];
    stage_dtb<false, KD>(dtb_lds, dt_bias, h, KD);
    wave_lds_sync();

    const size_t row_elems = (size_t)H * KD;
    const size_t base = ((size_t)t0 * H + h) * KD;
    const __amdgpu_buffer_rsrc_t sg = make_rsrc(g + base, (uint32_t)(((size_t)(len - 1) * row_elems + KD) * 2));
    const __amdgpu_buffer_rsrc_t sb = make_rsrc(beta + (size_t)t0 * H + h, (uint32_t)(((size_t)(len - 1) * H + 1) * 2));
    const uint32_t logit = __builtin_amdgcn_raw_buffer_load_b16(sb, tok * H * 2, 0, 0);
    if (grp == 0 && live) beta_out[(size_t)(t0 + tok) * H + h] = beta_sigmoid(logit);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        const int off = (int)((tok * row_elems + 32 * kb + 8 * grp) * 2);
        const u32x4_t g8 = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sg, off, 0, 0));
        float G[8];
        if (A > 0.f) {
            gate_cumsum(G, g8, dtb_lds, kb, grp, A, lb2, live);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) G[i] = 0.f;
        }
        if (live) {
            float *dst = G_out + base + tok * row_elems + 32 * kb + 8 * grp;
            *(f32x4_t *)dst = *(const f32x4_t *)&G[0];
            *(f32x4_t *)(dst + 4) = *(const f32x4_t *)&G[4];
        }
    }
}

}  // namespace

hipError_t launch_gate(const uint16_t *g, const uint16_t *beta, const float *A_log,
                       const float *dt_bias, float lower_bound, const int32_t *cu, int N, int T,
                       int H, int K, int64_t num_slots, float *G_out, float *beta_out,
                       hipStream_t stream)
{
    if (num_slots <= 0) return hipSuccess;
    dim3 grid((unsigned)(num_slots * H));
    const float lb2 = lower_bound * LOG2E;
#define KDA_GATE(KD_)                                                                     \
    hipLaunchKernelGGL((gate_kernel<KD_>), grid, dim3(64), 0, stream, g, beta, A_log,     \
                       dt_bias, lb2, cu, N, T, H, G_out, beta_out)
    if (K == HD) KDA_GATE(HD);
    else if (K == 2 * HD) KDA_GATE(2 * HD);
    else KDA_GATE(64);
#undef KDA_GATE
    return hipGetLastError();
}

hipError_t launch_intra(const uint16_t *q, const uint16_t *k, const uint16_t *g,
                        const uint16_t *beta, const float *A_log, const float *dt_bias,
                        float lower_bound, const int32_t *cu, int N, int T, int H, int K,
                        int64_t num_slots, uint8_t *ws, hipStream_t stream, bool scalar_gate)
{
    if (num_slots <= 0) return hipSuccess;
    dim3 grid((unsigned)(num_slots * H));
    const float lb2 = lower_bound * LOG2E;
#define KDA_INTRA(SG_, KD_)                                                               \
    hipLaunchKernelGGL((intra_kernel<SG_, KD_>), grid, dim3(64), 0, stream,              \
                       q, k, g, beta, A_log, dt_bias, lb2, cu, N, T, H, ws)
    if (K == HD) {
        if (scalar_gate) KDA_INTRA(true, HD); else KDA_INTRA(false, HD);
    } else if (K == 2 * HD) {
        if (scalar_gate) KDA_INTRA(true, 2 * HD); else KDA_INTRA(false, 2 * HD);
    } else {
        if (scalar_gate) KDA_INTRA(true, 64); else KDA_INTRA(false, 64);
    }
#undef KDA_INTRA
    return hipGetLastError();
}

}  // namespace kda
