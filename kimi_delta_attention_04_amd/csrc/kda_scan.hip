// Inter-chunk scan: the sequential part of the chunkwise algorithm.
//
// One wave owns one (sequence, head, 16-column slice of V).  Columns of the
// state evolve independently (each column sees the same transition and its
// own v entries), so the eight slices of a head need no communication.  The
// 128 x 16 fp32 state slice stays in MFMA accumulators for the whole
// sequence (8 tiles of 16 x 16); the row permutation of the tiles (see
// kda_device.h) makes the accumulators of tile pair (2kb, 2kb+1), rounded to
// bf16, exactly the B operand of the next chunk's 16x16x32 MFMAs, so the
// state never goes through LDS.  Per chunk:
//   P  = Kt S            X = V - P            E = T diag(beta) X
//   O  = scale (Qt S + Aqk E)  -> bf16 out
//   S  = diag(gamma) (S + Kb^T E)
// The long serial chain is what the FlashKDA write-up calls the low-
// parallelism second stage ("Moonshot AI Open-Sources FlashKDA", section
// "What makes the kernel fast"); here it is spread over (sequence, head,
// slice) waves instead of one block per head.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

struct ChunkOps {
    u32x4_t kt[4], qt[4], kb[4], ta;
    f32x4_t gam[8];
};

__device__ __forceinline__ void load_ops(ChunkOps &o, const uint8_t *rec, int l, int grp) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        o.kt[kb] = *(const u32x4_t *)(rec + REC_KT + (kb * 64 + l) * 16);
        o.qt[kb] = *(const u32x4_t *)(rec + REC_QT + (kb * 64 + l) * 16);
        o.kb[kb] = *(const u32x4_t *)(rec + REC_KB + (kb * 64 + l) * 16);
    }
    o.ta = *(const u32x4_t *)(rec + REC_TA + l * 16);
    const float *gp = (const float *)(rec + REC_GAM);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        o.gam[2 * kb] = *(const f32x4_t *)(gp + 32 * kb + 8 * grp);
        o.gam[2 * kb + 1] = *(const f32x4_t *)(gp + 32 * kb + 8 * grp + 4);
    }
}

__device__ __forceinline__ u32x2_t lo2(u32x4_t v) { u32x2_t r = {v[0], v[1]}; return r; }
__device__ __forceinline__ u32x2_t hi2(u32x4_t v) { u32x2_t r = {v[2], v[3]}; return r; }

__global__ __launch_bounds__(64) void scan_kernel(
    const uint16_t *__restrict__ v, const uint8_t *__restrict__ ws,
    const int32_t *__restrict__ cu, int N, int T, int H, float scale,
    const void *__restrict__ init, int init_fp32,
    void *__restrict__ fin, int fin_fp32, uint16_t *__restrict__ out)
{
    // Block b -> unit u (sequence, head) and slice s such that the eight
    // slices of a unit share b mod 8, i.e. the same XCD and L2.
    const int b = blockIdx.x;
    const int u = 8 * (b >> 6) + (b & 7);
    const int s = (b >> 3) & 7;
    if (u >= N * H) return;
    const int n = u / H, h = u % H;
    const int l = threadIdx.x;
    const int grp = l >> 4, cg = l & 15;
    const int col = 16 * s + cg;

    int64_t start, end;
    seq_range(cu, n, T, start, end);
    const int64_t L = end - start;
    const int nch = (int)((L + CS - 1) / CS);
    const int64_t slot0 = seq_slot0(cu, n, T);
    const size_t state_base = ((size_t)n * H + h) * HD * HD;

    // ---- state slice: S[t][j] = state[chan(t, 4grp+j)][col] ----------------
    f32x4_t S[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const size_t idx = state_base + (size_t)state_chan(t, 4 * grp + j) * HD + col;
            float x = 0.f;
            if (init) x = init_fp32 ? ((const float *)init)[idx] : bf16f(((const uint16_t *)init)[idx]);
            S[t][j] = x;
        }

    ChunkOps cur, nxt;
    if (nch > 0) load_ops(cur, ws + ((size_t)slot0 * H + h) * REC_BYTES, l, grp);

    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch) load_ops(nxt, ws + ((size_t)(slot0 + c + 1) * H + h) * REC_BYTES, l, grp);

        const int64_t tb = start + (int64_t)c * CS;
        const int len = (int)min((int64_t)CS, end - tb);
        float vv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * grp + j;
            vv[j] = r < len ? bf16f(v[((size_t)(tb + r) * H + h) * HD + col]) : 0.f;
        }

        // bf16 copy of the state as B operand: k-slots 8grp..8grp+7 of pair kb
        u32x4_t Sb[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            Sb[kb][0] = pack2(S[2 * kb][0], S[2 * kb][1]);
            Sb[kb][1] = pack2(S[2 * kb][2], S[2 * kb][3]);
            Sb[kb][2] = pack2(S[2 * kb + 1][0], S[2 * kb + 1][1]);
            Sb[kb][3] = pack2(S[2 * kb + 1][2], S[2 * kb + 1][3]);
        }
        f32x4_t P = {0.f, 0.f, 0.f, 0.f}, Qs = P;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            P = mfma_k32(cur.kt[kb], Sb[kb], P);
            Qs = mfma_k32(cur.qt[kb], Sb[kb], Qs);
        }
        u32x2_t Xb;
        Xb[0] = pack2(vv[0] - P[0], vv[1] - P[1]);
        Xb[1] = pack2(vv[2] - P[2], vv[3] - P[3]);
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4_t E = mfma_k16(lo2(cur.ta), Xb, zero);
        u32x2_t Eb;
        Eb[0] = pack2(E[0], E[1]);
        Eb[1] = pack2(E[2], E[3]);
        const f32x4_t O = mfma_k16(hi2(cur.ta), Eb, Qs);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * grp + j;
            if (r < len) out[((size_t)(tb + r) * H + h) * HD + col] = tobf16(scale * O[j]);
        }
#pragma unroll
        for (int tp = 0; tp < 4; ++tp) {
            S[2 * tp] = mfma_k16(lo2(cur.kb[tp]), Eb, S[2 * tp]);
            S[2 * tp + 1] = mfma_k16(hi2(cur.kb[tp]), Eb, S[2 * tp + 1]);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = S[t] * cur.gam[t];
        if (c + 1 < nch) cur = nxt;
    }

    if (fin) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const size_t idx = state_base + (size_t)state_chan(t, 4 * grp + j) * HD + col;
                if (fin_fp32) ((float *)fin)[idx] = S[t][j];
                else ((uint16_t *)fin)[idx] = tobf16(S[t][j]);
            }
    }
}

}  // namespace

hipError_t launch_scan(const uint16_t *v, const uint8_t *ws, const int32_t *cu, int N, int T,
                       int H, float scale, const void *init, int init_fp32, void *fin,
                       int fin_fp32, uint16_t *out, hipStream_t stream)
{
    const int64_t units = (int64_t)N * H;
    const int64_t blocks = 64 * ((units + 7) / 8);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(scan_kernel, dim3((unsigned)blocks), dim3(64), 0, stream,
                       v, ws, cu, N, T, H, scale, init, init_fp32, fin, fin_fp32, out);
    return hipGetLastError();
}

}  // namespace kda
