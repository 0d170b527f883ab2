// Decode step: one new token per sequence applied to the recurrent state in
// place, the step that follows a prefill and consumes its final state
// ("FlashKDA" product page, Main Features: the recurrent state carried
// between prefill and decode; "Moonshot AI Rilis FlashKDA", the initial and
// final state arguments).  Per (sequence n, head h), with the state S
// (K x V, row-major, V contiguous) of that pair:
//
//   alpha[c] = exp(max(-exp(A_log[h]) softplus(g[c] + dt_bias[h K + c]), lower_bound))
//   S        = Diag(alpha) S
//   S        = S + beta k (v - S^T k)^T          (beta = sigmoid(logit))
//   o        = scale S^T q
//
// which is the token recurrence of the prefill for a single token.
//
// One workgroup of D^2 / 64 threads per (sequence, head), head dimension
// K = V = D (64, 128 or 256: 64, 256 or 1024 threads).  Thread t holds the
// 16 x 4 block of the state at rows 16 (t / (D/4)) .. +15 and columns
// 4 (t % (D/4)) .. +3 in registers: each state row is read and written by
// D/4 consecutive lanes as one contiguous row.  The two contractions over
// rows (S^T k, S^T q) are summed per thread over its 16 rows and then over
// the D/16 row groups through LDS, in a fixed order.  The step moves the
// whole state through HBM twice (read and write), so it is HBM-bound:
// 128 KiB per (sequence, head) for an fp32 state at D = 128.  The updated
// state is written with non-temporal stores: a batch of states is larger
// than the memory-side cache, and written the normal way it sits there
// dirty and is written back under the next step's reads (measured at
// 64 sequences x 96 heads: 0.151 -> 0.121 ms per step).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

template <int D> constexpr int DEC_THREADS = D * D / 64;

template <bool F32, int D>
__global__ __launch_bounds__(DEC_THREADS<D>) void decode_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ g,
    const uint16_t *__restrict__ beta, float scale, const float *__restrict__ A_log,
    const float *__restrict__ dt_bias, float lb2, int H, void *__restrict__ state,
    uint16_t *__restrict__ out)
{
    constexpr int CG = D / 4;                    // column groups of 4 columns
    constexpr int RG = D / 16;                   // row groups of 16 rows
    static_assert(CG * RG == DEC_THREADS<D>, "one 16 x 4 block per thread");
    const int u = blockIdx.x;                    // (n, h) pair, n-major
    const int h = u % H;
    const int t = threadIdx.x;
    const int cgp = t % CG, rg = t / CG;
    __shared__ float kk[D], qq[D], al[D];
    __shared__ f32x4_t part[RG][CG];
    const size_t vec = (size_t)u * D;

    // per-channel decay in base 2 and the key / query vectors
    if (t < D) {
        const float A = expf(A_log[h]);
        float la2 = 0.f;                         // A = 0 (A_log = -inf): no decay
        if (A > 0.f) {
            const float x2 = bf16f(g[vec + t]) * LOG2E +
                             (dt_bias ? dt_bias[(size_t)h * D + t] * LOG2E : 0.f);
            la2 = fmaxf(-A * fast_log2(1.f + fast_exp2(x2)), lb2);
        }
        al[t] = fast_exp2(la2);
        kk[t] = bf16f(k[vec + t]);
        qq[t] = bf16f(q[vec + t]);
    }
    const float b = __builtin_amdgcn_rcpf(1.f + fast_exp2(-bf16f(beta[u]) * LOG2E));
    __syncthreads();

    // this thread's 16 x 4 block of the state
    const size_t base = (size_t)u * D * D + (size_t)(16 * rg) * D + 4 * cgp;
    float S[16][4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        if (F32) {
            const f32x4_t x = *(const f32x4_t *)((const float *)state + base + (size_t)r * D);
#pragma unroll
            for (int c = 0; c < 4; ++c) S[r][c] = x[c];
        } else {
            const u32x2_t x = *(const u32x2_t *)((const uint16_t *)state + base + (size_t)r * D);
            S[r][0] = bf16lo(x[0]); S[r][1] = bf16hi(x[0]);
            S[r][2] = bf16lo(x[1]); S[r][3] = bf16hi(x[1]);
        }
    }

    // S = Diag(alpha) S, then partial (S^T k) over this thread's rows
    f32x4_t pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float a = al[16 * rg + r], kr = kk[16 * rg + r];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            S[r][c] *= a;
            pu[c] += S[r][c] * kr;
        }
    }
    part[rg][cgp] = pu;
    __syncthreads();
    f32x4_t su = part[0][cgp];
#pragma unroll
    for (int j = 1; j < RG; ++j) su += part[j][cgp];
    const u32x2_t vw = *(const u32x2_t *)(v + vec + 4 * cgp);
    const float vv[4] = {bf16lo(vw[0]), bf16hi(vw[0]), bf16lo(vw[1]), bf16hi(vw[1])};
    float d[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) d[c] = b * (vv[c] - su[c]);
    __syncthreads();                             // every thread has read part

    // S += k d^T, partial (S^T q), state written back in place
    f32x4_t po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float kr = kk[16 * rg + r], qr = qq[16 * rg + r];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            S[r][c] += kr * d[c];
            po[c] += S[r][c] * qr;
        }
        if (F32) {
            const f32x4_t x = {S[r][0], S[r][1], S[r][2], S[r][3]};
            __builtin_nontemporal_store(x, (f32x4_t *)((float *)state + base + (size_t)r * D));
        } else {
            const u32x2_t x = {pack2(S[r][0], S[r][1]), pack2(S[r][2], S[r][3])};
            __builtin_nontemporal_store(x, (u32x2_t *)((uint16_t *)state + base + (size_t)r * D));
        }
    }
    part[rg][cgp] = po;
    __syncthreads();
    if (rg == 0) {
        f32x4_t so = part[0][cgp];
#pragma unroll
        for (int j = 1; j < RG; ++j) so += part[j][cgp];
        const u32x2_t o = {pack2(scale * so[0], scale * so[1]), pack2(scale * so[2], scale * so[3])};
        *(u32x2_t *)(out + vec + 4 * cgp) = o;
    }
}

}  // namespace

hipError_t launch_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const uint16_t *g, const uint16_t *beta, float scale,
                         const float *A_log, const float *dt_bias, float lower_bound, int N,
                         int H, int D, void *state, int state_fp32, uint16_t *out,
                         hipStream_t stream)
{
    const unsigned blocks = (unsigned)((int64_t)N * H);
    if (blocks == 0) return hipSuccess;
    const float lb2 = lower_bound * LOG2E;
#define KDA_DECODE(F32_, D_)                                                                  \
    hipLaunchKernelGGL((decode_kernel<F32_, D_>), dim3(blocks), dim3(DEC_THREADS<D_>), 0, stream, \
                       q, k, v, g, beta, scale, A_log, dt_bias, lb2, H, state, out)
    if (D == 64) {
        if (state_fp32) KDA_DECODE(true, 64); else KDA_DECODE(false, 64);
    } else if (D == 256) {
        if (state_fp32) KDA_DECODE(true, 256); else KDA_DECODE(false, 256);
    } else {
        if (state_fp32) KDA_DECODE(true, 128); else KDA_DECODE(false, 128);
    }
#undef KDA_DECODE
    return hipGetLastError();
}

}  // namespace kda
