// C-ABI of libkda: argument validation, workspace, launches.
#include <math.h>
#include <stdlib.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include <hip/hip_runtime.h>

#include "kda.h"
#include "kda_device.h"
#include "kda_launch.h"

namespace {

// 16 tokens * |lower_bound| * log2(e) must stay below ~125 so that both
// 2^G and 2^-G of the in-chunk cumulative decay are normal fp32 / bf16.
constexpr float kLowerBoundMin = -5.4f;
constexpr int kMaxDevices = 64;

// Workspace memory the library's pool keeps reserved across calls once the
// stream that freed it has synchronised; anything above is returned to the
// device (kda_trim_workspace releases the rest on demand).
constexpr uint64_t kDefaultKeepBytes = 1ull << 30;

std::mutex g_pool_mu;
hipMemPool_t g_pools[kMaxDevices];
bool g_pool_ready[kMaxDevices];

kda_status_t device_pool(hipMemPool_t *pool, bool create = true) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_pool_mu);
    if (!g_pool_ready[dev]) {
        if (!create) { *pool = nullptr; return KDA_OK; }
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p = nullptr;
        if (hipMemPoolCreate(&p, &props) != hipSuccess) return KDA_ERR_LAUNCH;
        uint64_t keep = kDefaultKeepBytes;   // freed blocks up to this are kept for later calls
        if (hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep) != hipSuccess) {
            (void)hipMemPoolDestroy(p);
            return KDA_ERR_LAUNCH;
        }
        g_pools[dev] = p;
        g_pool_ready[dev] = true;
    }
    *pool = g_pools[dev];
    return KDA_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Optional per-thread stage events (kda_set_stage_events).
thread_local hipEvent_t t_stage_events[3] = {nullptr, nullptr, nullptr};
thread_local hipEvent_t t_bwd_events[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};

hipError_t mark(int i, hipStream_t s) {
    return t_stage_events[i] ? hipEventRecord(t_stage_events[i], s) : hipSuccess;
}

// 16-token chunk slots: floor(B T / 16) + N
int64_t num_slots(int32_t B, int32_t T, int32_t N) {
    return ((int64_t)B * T) / kda::CS + N;
}

kda_status_t check_sizes(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                         const int32_t *cu, int32_t N) {
    if (B < 1 || T < 0 || H < 1 || N < 1) return KDA_ERR_INVALID_ARG;
    if (cu ? (B != 1) : (N != B)) return KDA_ERR_INVALID_ARG;
    // K = V = 64, 128 or 256
    if (K != V || (K != kda::HD && K != 2 * kda::HD && K != 64)) return KDA_ERR_UNSUPPORTED;
    // token-row and unit counts must fit the int32 grid / index arithmetic
    if ((int64_t)B * T > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    if (num_slots(B, T, N) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    // one intra workgroup per (chunk slot, head) in a 1-D grid
    if (num_slots(B, T, N) * H > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)N * H > INT32_MAX / 64) return KDA_ERR_UNSUPPORTED;
    // byte offsets within one chunk's 16 token rows of all heads are 32-bit
    if ((int64_t)H * (K > kda::HD ? K : kda::HD) * 2 * kda::CS > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

// Opt-in device check of the cu_seqlens contents (KDA_CHECK_CU_SEQLENS set
// to a value other than "0" in the environment): cu[0] = 0, non-decreasing,
// cu[N] = T.  One workgroup; the result is copied back to the host, so the
// call synchronises with the stream (a debugging aid, off by default).
__global__ void check_cu_kernel(const int32_t *__restrict__ cu, int N, int T, int *__restrict__ bad) {
    int b = 0;
    for (int i = threadIdx.x; i < N; i += blockDim.x)
        if (cu[i + 1] < cu[i]) b = 1;
    if (threadIdx.x == 0 && (cu[0] != 0 || cu[N] != T)) b = 1;
    b = __syncthreads_or(b);
    if (threadIdx.x == 0) *bad = b;
}

bool cu_check_enabled() {
    const char *e = getenv("KDA_CHECK_CU_SEQLENS");
    return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

// KDA_OK, KDA_ERR_INVALID_ARG for bad contents, or KDA_ERR_LAUNCH.  `bad`:
// one device int the check may overwrite.
kda_status_t check_cu_flag(const int32_t *cu, int N, int T, hipStream_t s, int *bad) {
    int host_bad = 1;
    hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, s, cu, N, T, bad);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(&host_bad, bad, sizeof(int), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return KDA_ERR_LAUNCH;
    return host_bad ? KDA_ERR_INVALID_ARG : KDA_OK;
}

kda_status_t check_cu_contents(const int32_t *cu, int N, int T, hipStream_t s, hipMemPool_t pool) {
    int *bad = nullptr;
    if (hipMallocFromPoolAsync((void **)&bad, sizeof(int), pool, s) != hipSuccess || !bad) {
        (void)hipGetLastError();
        return KDA_ERR_OUT_OF_MEMORY;
    }
    kda_status_t st = check_cu_flag(cu, N, T, s, bad);
    if (hipFreeAsync(bad, s) != hipSuccess && st == KDA_OK) st = KDA_ERR_LAUNCH;
    return st;
}

kda_status_t check_gate(float lower_bound) {
    if (!isfinite(lower_bound) || lower_bound > 0.f) return KDA_ERR_INVALID_ARG;
    if (lower_bound < kLowerBoundMin) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH";
        case KDA_ERR_OUT_OF_MEMORY: return "KDA_ERR_OUT_OF_MEMORY";
    }
    return "KDA_ERR_UNKNOWN";
}

float kda_lower_bound_min(void) { return kLowerBoundMin; }

int32_t kda_chunk_size(void) { return kda::CS; }

kda_status_t kda_trim_workspace(size_t keep_bytes) {
    hipMemPool_t pool = nullptr;
    kda_status_t st = device_pool(&pool, false);
    if (st != KDA_OK || !pool) return st;
    return hipMemPoolTrimTo(pool, keep_bytes) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

size_t kda_workspace_reserved(void) {
    hipMemPool_t pool = nullptr;
    if (device_pool(&pool, false) != KDA_OK || !pool) return 0;
    uint64_t v = 0;
    if (hipMemPoolGetAttribute(pool, hipMemPoolAttrReservedMemCurrent, &v) != hipSuccess) return 0;
    return (size_t)v;
}

size_t kda_record_workspace_size(int32_t B, int32_t T, int32_t H, int32_t num_seqs, int32_t K) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 1) return 0;
    if (K != 64 && K != kda::HD && K != 2 * kda::HD) return 0;
    const size_t rec = (size_t)kda::rec_bytes_for(K);
    return (size_t)num_slots(B, T, num_seqs) * (size_t)H * rec;
}

size_t kda_workspace_size(int32_t B, int32_t T, int32_t H, int32_t num_seqs) {
    return kda_workspace_size_hd(B, T, H, num_seqs, kda::HD);
}

size_t kda_workspace_size_hd(int32_t B, int32_t T, int32_t H, int32_t num_seqs, int32_t K) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 1) return 0;
    if (K != 64 && K != kda::HD && K != 2 * kda::HD) return 0;
    return kda_record_workspace_size(B, T, H, num_seqs, K);
}

}  // extern "C"

namespace {

// Argument checks shared by the forward entry points (before any HIP call).
kda_status_t fwd_validate(const void *q, const void *k, const void *v, const void *g,
                          const void *beta, float scale, const float *A_log,
                          const float *dt_bias, float lower_bound, const int32_t *cu_seqlens,
                          int32_t num_seqs, const void *initial_state,
                          kda_dtype_t initial_state_dtype, const void *final_state,
                          kda_dtype_t final_state_dtype, const void *out, int32_t B, int32_t T,
                          int32_t H, int32_t K, int32_t V, bool scalar_gate)
{
    // With no tokens the token buffers are never touched and may be NULL.
    const bool no_tokens = (int64_t)B * T == 0;
    if (!A_log) return KDA_ERR_INVALID_ARG;
    if (!no_tokens && (!q || !k || !v || !g || !beta || !out)) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, scalar_gate ? 2 : 16) ||
        !aligned(out, 16) || !aligned(beta, 2) || !aligned(A_log, 4) ||
        !aligned(dt_bias, 4) || !aligned(cu_seqlens, 4) || !aligned(initial_state, 16) ||
        !aligned(final_state, 16))
        return KDA_ERR_INVALID_ARG;
    if ((initial_state_dtype != KDA_DTYPE_BF16 && initial_state_dtype != KDA_DTYPE_FP32) ||
        (final_state_dtype != KDA_DTYPE_BF16 && final_state_dtype != KDA_DTYPE_FP32))
        return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    kda_status_t st = check_sizes(B, T, H, K, V, cu_seqlens, num_seqs);
    if (st != KDA_OK) return st;
    return check_gate(lower_bound);
}

// The forward's kernels on stream s with the workspace ws of
// kda_workspace_size_hd(B, T, H, num_seqs, K) bytes.
hipError_t fwd_launch(const void *q, const void *k, const void *v, const void *g,
                      const void *beta, float scale, const float *A_log, const float *dt_bias,
                      float lower_bound, const int32_t *cu_seqlens, int32_t num_seqs,
                      const void *initial_state, kda_dtype_t initial_state_dtype,
                      void *final_state, kda_dtype_t final_state_dtype, void *out, int32_t B,
                      int32_t T, int32_t H, int32_t K, int32_t V, hipStream_t s,
                      bool scalar_gate, void *ws)
{
    const int64_t slots = num_slots(B, T, num_seqs);
    const int init32 = initial_state_dtype == KDA_DTYPE_FP32;
    const int fin32 = final_state_dtype == KDA_DTYPE_FP32;
    hipError_t e = mark(0, s);
    if (e == hipSuccess)
        e = kda::launch_intra((const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)g,
                              (const uint16_t *)beta, A_log, dt_bias, lower_bound, cu_seqlens,
                              num_seqs, T, H, K, slots, (uint8_t *)ws, s, scalar_gate);
    if (e == hipSuccess) e = mark(1, s);
    if (e == hipSuccess)
        e = kda::launch_scan((const uint16_t *)v, (const uint8_t *)ws, cu_seqlens, num_seqs, T, H, K,
                             V, scale, initial_state, init32, final_state, fin32, (uint16_t *)out, s);
    if (e == hipSuccess) e = mark(2, s);
    return e;
}

// kda_fwd and kda_fwd_scalar_gate: scalar_gate selects the layout of g
// ([B, T, H, K] or [B, T, H]) and dt_bias ([H*K] or [H]).
kda_status_t fwd_impl(const void *q, const void *k, const void *v, const void *g,
                      const void *beta, float scale,
                      const float *A_log, const float *dt_bias, float lower_bound,
                      const int32_t *cu_seqlens, int32_t num_seqs,
                      const void *initial_state, kda_dtype_t initial_state_dtype,
                      void *final_state, kda_dtype_t final_state_dtype,
                      void *out,
                      int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                      void *stream, bool scalar_gate)
{
    kda_status_t st = fwd_validate(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
                                   cu_seqlens, num_seqs, initial_state, initial_state_dtype,
                                   final_state, final_state_dtype, out, B, T, H, K, V, scalar_gate);
    if (st != KDA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const size_t bytes = kda_workspace_size_hd(B, T, H, num_seqs, K);
    hipMemPool_t pool;
    if ((st = device_pool(&pool)) != KDA_OK) return st;
    if (cu_seqlens && cu_check_enabled() &&
        (st = check_cu_contents(cu_seqlens, num_seqs, (int)((int64_t)B * T), s, pool)) != KDA_OK)
        return st;
    void *ws = nullptr;
    if (hipMallocFromPoolAsync(&ws, bytes, pool, s) != hipSuccess || !ws) {
        (void)hipGetLastError();
        return KDA_ERR_OUT_OF_MEMORY;
    }
    const hipError_t e = fwd_launch(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
                                    cu_seqlens, num_seqs, initial_state, initial_state_dtype,
                                    final_state, final_state_dtype, out, B, T, H, K, V, s,
                                    scalar_gate, ws);
    const hipError_t ef = hipFreeAsync(ws, s);
    if (e != hipSuccess || ef != hipSuccess) return KDA_ERR_LAUNCH;
    return KDA_OK;
}


kda_status_t bwd_launch_all(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, float scale, const float *A_log,
                            const float *dt_bias, float lower_bound, const int32_t *cu_seqlens,
                            int32_t num_seqs, const void *initial_state,
                            kda_dtype_t initial_state_dtype, const void *d_out,
                            const float *d_final_state, void *dq, void *dk, void *dv, void *dg,
                            void *dbeta, float *dA_log, float *ddt_bias, float *d_initial_state,
                            int32_t B, int32_t T, int32_t H, int32_t K, void *stream,
                            uint16_t *dg_scalar);

}  // namespace

extern "C" {

kda_status_t kda_fwd(const void *q, const void *k, const void *v, const void *g,
                     const void *beta, float scale,
                     const float *A_log, const float *dt_bias, float lower_bound,
                     const int32_t *cu_seqlens, int32_t num_seqs,
                     const void *initial_state, kda_dtype_t initial_state_dtype,
                     void *final_state, kda_dtype_t final_state_dtype,
                     void *out,
                     int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                     void *stream)
{
    return fwd_impl(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, cu_seqlens, num_seqs,
                    initial_state, initial_state_dtype, final_state, final_state_dtype, out,
                    B, T, H, K, V, stream, false);
}

kda_status_t kda_fwd_scalar_gate(const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, float scale,
                                 const float *A_log, const float *dt_bias, float lower_bound,
                                 const int32_t *cu_seqlens, int32_t num_seqs,
                                 const void *initial_state, kda_dtype_t initial_state_dtype,
                                 void *final_state, kda_dtype_t final_state_dtype,
                                 void *out,
                                 int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                 void *stream)
{
    return fwd_impl(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, cu_seqlens, num_seqs,
                    initial_state, initial_state_dtype, final_state, final_state_dtype, out,
                    B, T, H, K, V, stream, true);
}

kda_status_t kda_debug_gate(const void *g, const void *beta,
                            const float *A_log, const float *dt_bias, float lower_bound,
                            const int32_t *cu_seqlens, int32_t num_seqs,
                            float *G, float *beta_out,
                            int32_t B, int32_t T, int32_t H, int32_t K, void *stream)
{
    const bool no_tokens = (int64_t)B * T == 0;
    if (!A_log || (!no_tokens && (!g || !beta || !G || !beta_out))) return KDA_ERR_INVALID_ARG;
    if (!aligned(g, 16) || !aligned(G, 16) || !aligned(beta, 2) || !aligned(beta_out, 4) ||
        !aligned(A_log, 4) || !aligned(dt_bias, 4) || !aligned(cu_seqlens, 4))
        return KDA_ERR_INVALID_ARG;
    kda_status_t st = check_sizes(B, T, H, K, K, cu_seqlens, num_seqs);
    if (st != KDA_OK) return st;
    if ((st = check_gate(lower_bound)) != KDA_OK) return st;
    if (no_tokens) return KDA_OK;
    const hipError_t e =
        kda::launch_gate((const uint16_t *)g, (const uint16_t *)beta, A_log, dt_bias, lower_bound,
                         cu_seqlens, num_seqs, T, H, K, num_slots(B, T, num_seqs), G, beta_out,
                         (hipStream_t)stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_debug_intra(const void *q, const void *k, const void *g,
                             const void *beta,
                             const float *A_log, const float *dt_bias, float lower_bound,
                             const int32_t *cu_seqlens, int32_t num_seqs,
                             int32_t B, int32_t T, int32_t H, int32_t K,
                             void *workspace, void *stream)
{
    if (!q || !k || !g || !beta || !A_log || !workspace) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(g, 16) || !aligned(workspace, 16) ||
        !aligned(beta, 2) || !aligned(A_log, 4) || !aligned(dt_bias, 4) ||
        !aligned(cu_seqlens, 4))
        return KDA_ERR_INVALID_ARG;
    kda_status_t st = check_sizes(B, T, H, K, K, cu_seqlens, num_seqs);
    if (st != KDA_OK) return st;
    if ((st = check_gate(lower_bound)) != KDA_OK) return st;
    const hipError_t e =
        kda::launch_intra((const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)g,
                          (const uint16_t *)beta, A_log, dt_bias, lower_bound, cu_seqlens, num_seqs,
                          T, H, K, num_slots(B, T, num_seqs), (uint8_t *)workspace,
                          (hipStream_t)stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_debug_scan_step(const void *v, const void *records, const int32_t *cu_seqlens,
                                 int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                                 int32_t V, float scale, const void *initial_state,
                                 kda_dtype_t initial_state_dtype, void *final_state,
                                 kda_dtype_t final_state_dtype, void *out, int32_t part_cols,
                                 void *stream)
{
    const bool no_tokens = (int64_t)B * T == 0;
    if (!records || (!no_tokens && (!v || !out))) return KDA_ERR_INVALID_ARG;
    if (!aligned(v, 16) || !aligned(records, 16) || !aligned(out, 16) ||
        !aligned(cu_seqlens, 4) || !aligned(initial_state, 16) || !aligned(final_state, 16))
        return KDA_ERR_INVALID_ARG;
    if ((initial_state_dtype != KDA_DTYPE_BF16 && initial_state_dtype != KDA_DTYPE_FP32) ||
        (final_state_dtype != KDA_DTYPE_BF16 && final_state_dtype != KDA_DTYPE_FP32))
        return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    kda_status_t st = check_sizes(B, T, H, K, V, cu_seqlens, num_seqs);
    if (st != KDA_OK) return st;
    if (part_cols != 0 && part_cols != 32 && part_cols != 64 && part_cols != 128)
        return KDA_ERR_INVALID_ARG;
    if (part_cols > V) return KDA_ERR_INVALID_ARG;
    const hipError_t e = kda::launch_scan(
        (const uint16_t *)v, (const uint8_t *)records, cu_seqlens, num_seqs, T, H, K, V, scale,
        initial_state, initial_state_dtype == KDA_DTYPE_FP32, final_state,
        final_state_dtype == KDA_DTYPE_FP32, (uint16_t *)out, (hipStream_t)stream, part_cols);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_decode(const void *q, const void *k, const void *v, const void *g,
                        const void *beta, float scale,
                        const float *A_log, const float *dt_bias, float lower_bound,
                        void *state, kda_dtype_t state_dtype, void *out,
                        int32_t N, int32_t H, int32_t K, int32_t V, void *stream)
{
    if (!q || !k || !v || !g || !beta || !A_log || !state || !out) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) ||
        !aligned(out, 16) || !aligned(state, 16) || !aligned(beta, 2) || !aligned(A_log, 4) ||
        !aligned(dt_bias, 4))
        return KDA_ERR_INVALID_ARG;
    if (state_dtype != KDA_DTYPE_BF16 && state_dtype != KDA_DTYPE_FP32) return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !isfinite(lower_bound) || lower_bound > 0.f) return KDA_ERR_INVALID_ARG;
    if (N < 1 || H < 1) return KDA_ERR_INVALID_ARG;
    if (K != V || (K != 64 && K != kda::HD && K != 2 * kda::HD)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)N * H > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    hipError_t e = kda::launch_decode((const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v,
                                      (const uint16_t *)g, (const uint16_t *)beta, scale, A_log,
                                      dt_bias, lower_bound, N, H, K, state,
                                      state_dtype == KDA_DTYPE_FP32, (uint16_t *)out,
                                      (hipStream_t)stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_bwd(const void *q, const void *k, const void *v, const void *g,
                     const void *beta, float scale,
                     const float *A_log, const float *dt_bias, float lower_bound,
                     const int32_t *cu_seqlens, int32_t num_seqs,
                     const void *initial_state, kda_dtype_t initial_state_dtype,
                     const void *d_out, const float *d_final_state,
                     void *dq, void *dk, void *dv, void *dg, void *dbeta,
                     float *dA_log, float *ddt_bias, float *d_initial_state,
                     int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, void *stream)
{
    const bool no_tokens = (int64_t)B * T == 0;
    if (!A_log || !dA_log) return KDA_ERR_INVALID_ARG;
    if (!no_tokens && (!q || !k || !v || !g || !beta || !d_out || !dq || !dk || !dv || !dg ||
                       !dbeta))
        return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) ||
        !aligned(d_out, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(dg, 16) || !aligned(beta, 2) || !aligned(dbeta, 2) || !aligned(A_log, 4) ||
        !aligned(dt_bias, 4) || !aligned(dA_log, 4) || !aligned(ddt_bias, 4) ||
        !aligned(cu_seqlens, 4) || !aligned(initial_state, 16) ||
        !aligned(d_final_state, 16) || !aligned(d_initial_state, 16))
        return KDA_ERR_INVALID_ARG;
    if (initial_state_dtype != KDA_DTYPE_BF16 && initial_state_dtype != KDA_DTYPE_FP32)
        return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    kda_status_t st = check_sizes(B, T, H, K, V, cu_seqlens, num_seqs);
    if (st != KDA_OK) return st;
    if (K != kda::HD && K != 64 && K != 2 * kda::HD) return KDA_ERR_UNSUPPORTED;   // K = V = 64, 128 or 256
    if ((st = check_gate(lower_bound)) != KDA_OK) return st;
    return bwd_launch_all(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, cu_seqlens,
                          num_seqs, initial_state, initial_state_dtype, d_out, d_final_state, dq,
                          dk, dv, dg, dbeta, dA_log, ddt_bias, d_initial_state, B, T, H, K, stream,
                          nullptr);
}

}  // extern "C"

namespace {

// The backward's workspace, the optional cu_seqlens check and its launches,
// for arguments already validated.  dg_scalar: see kda::launch_bwd.
kda_status_t bwd_launch_all(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, float scale, const float *A_log,
                            const float *dt_bias, float lower_bound, const int32_t *cu_seqlens,
                            int32_t num_seqs, const void *initial_state,
                            kda_dtype_t initial_state_dtype, const void *d_out,
                            const float *d_final_state, void *dq, void *dk, void *dv, void *dg,
                            void *dbeta, float *dA_log, float *ddt_bias, float *d_initial_state,
                            int32_t B, int32_t T, int32_t H, int32_t K, void *stream,
                            uint16_t *dg_scalar)
{
    kda_status_t st;
    hipStream_t s = (hipStream_t)stream;
    const int64_t slots = num_slots(B, T, num_seqs);
    const size_t bytes = kda::bwd_workspace_bytes(slots, H, K);
    hipMemPool_t pool;
    if ((st = device_pool(&pool)) != KDA_OK) return st;
    if (cu_seqlens && cu_check_enabled() &&
        (st = check_cu_contents(cu_seqlens, num_seqs, (int)((int64_t)B * T), s, pool)) != KDA_OK)
        return st;
    void *ws = nullptr;
    if (hipMallocFromPoolAsync(&ws, bytes, pool, s) != hipSuccess || !ws) {
        (void)hipGetLastError();
        return KDA_ERR_OUT_OF_MEMORY;
    }
    hipError_t e = kda::launch_bwd((const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v,
                                   (const uint16_t *)g, (const uint16_t *)beta, scale, A_log,
                                   dt_bias, lower_bound, cu_seqlens, num_seqs, T, H, K, slots,
                                   initial_state, initial_state_dtype == KDA_DTYPE_FP32,
                                   (const uint16_t *)d_out, d_final_state, (uint16_t *)dq,
                                   (uint16_t *)dk, (uint16_t *)dv, (uint16_t *)dg,
                                   (uint16_t *)dbeta, dA_log, ddt_bias, d_initial_state, ws, s,
                                   t_bwd_events, dg_scalar);
    hipError_t ef = hipFreeAsync(ws, s);
    if (e != hipSuccess || ef != hipSuccess) return KDA_ERR_LAUNCH;
    return KDA_OK;
}

// The Gated DeltaNet backward around the channel-wise one: its forward is
// the channel-wise forward with every key channel's gate input equal to the
// token's one value (and dt_bias[h] for every channel of head h), so its
// gradients are the channel-wise ones with the gate's and dt_bias's summed
// over the channels (the chunk kernel sums the gate's, kda::launch_bwd's
// dg_scalar).  gate_broadcast_kernel writes that channel-wise gate (one
// 16-byte piece of eight channels per thread, grid-stride) and dt_bias.
__global__ void gate_broadcast_kernel(const uint16_t *__restrict__ g, const float *__restrict__ dtb,
                                      int64_t pieces, int K, int H, uint16_t *__restrict__ gb,
                                      float *__restrict__ dtbb) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int per = K / 8;                                  // pieces per (token, head)
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pieces; i += stride) {
        const uint32_t w = g[i / per];
        const uint32_t two = w | (w << 16);
        uint4 v;
        v.x = v.y = v.z = v.w = two;
        *(uint4 *)(gb + 8 * i) = v;
    }
    if (dtbb)
        for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < (int64_t)H * K; j += stride)
            dtbb[j] = dtb[j / K];
}

// ddt[h] = sum over the channels of ddtb[h, c], in channel order (fp32).
__global__ void dtb_reduce_kernel(const float *__restrict__ ddtb, int H, int K,
                                  float *__restrict__ ddt) {
    for (int h = blockIdx.x * blockDim.x + threadIdx.x; h < H; h += gridDim.x * blockDim.x) {
        float acc = 0.f;
        for (int c = 0; c < K; ++c) acc += ddtb[(size_t)h * K + c];
        ddt[h] = acc;
    }
}

constexpr size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

kda_status_t kda_bwd_scalar_gate(const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, float scale,
                                 const float *A_log, const float *dt_bias, float lower_bound,
                                 const int32_t *cu_seqlens, int32_t num_seqs,
                                 const void *initial_state, kda_dtype_t initial_state_dtype,
                                 const void *d_out, const float *d_final_state,
                                 void *dq, void *dk, void *dv, void *dg, void *dbeta,
                                 float *dA_log, float *ddt_bias, float *d_initial_state,
                                 int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                 void *stream)
{
    const bool no_tokens = (int64_t)B * T == 0;
    if (!A_log || !dA_log) return KDA_ERR_INVALID_ARG;
    if (!no_tokens && (!q || !k || !v || !g || !beta || !d_out || !dq || !dk || !dv || !dg ||
                       !dbeta))
        return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 2) ||
        !aligned(d_out, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(dg, 2) || !aligned(beta, 2) || !aligned(dbeta, 2) || !aligned(A_log, 4) ||
        !aligned(dt_bias, 4) || !aligned(dA_log, 4) || !aligned(ddt_bias, 4) ||
        !aligned(cu_seqlens, 4) || !aligned(initial_state, 16) ||
        !aligned(d_final_state, 16) || !aligned(d_initial_state, 16))
        return KDA_ERR_INVALID_ARG;
    if (initial_state_dtype != KDA_DTYPE_BF16 && initial_state_dtype != KDA_DTYPE_FP32)
        return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    kda_status_t st = check_sizes(B, T, H, K, V, cu_seqlens, num_seqs);
    if (st != KDA_OK) return st;
    if ((st = check_gate(lower_bound)) != KDA_OK) return st;

    hipStream_t s = (hipStream_t)stream;
    const int64_t rows = (int64_t)B * T * H;                // (token, head) pairs
    const size_t gbytes = round256((size_t)rows * K * 2);
    const size_t hbytes = round256((size_t)H * K * 4);
    const size_t bytes = gbytes + (dt_bias ? hbytes : 0) + (ddt_bias ? hbytes : 0);
    hipMemPool_t pool;
    if ((st = device_pool(&pool)) != KDA_OK) return st;
    void *buf = nullptr;
    if (bytes > 0) {
        if (hipMallocFromPoolAsync(&buf, bytes, pool, s) != hipSuccess || !buf) {
            (void)hipGetLastError();
            return KDA_ERR_OUT_OF_MEMORY;
        }
    }
    uint8_t *p = (uint8_t *)buf;
    uint16_t *gb = (uint16_t *)p;                           // the gate, broadcast
    float *dtbb = dt_bias ? (float *)(p + gbytes) : nullptr;
    float *ddtb = ddt_bias ? (float *)(p + gbytes + (dt_bias ? hbytes : 0)) : nullptr;
    const unsigned blocks = (unsigned)std::min<int64_t>(4096, std::max<int64_t>(1, (rows * K / 8 + 255) / 256));
    kda_status_t r = KDA_OK;
    if (rows > 0 || dtbb) {
        hipLaunchKernelGGL(gate_broadcast_kernel, dim3(blocks), dim3(256), 0, s, (const uint16_t *)g,
                           dt_bias, rows * K / 8, K, H, gb, dtbb);
        if (hipGetLastError() != hipSuccess) r = KDA_ERR_LAUNCH;
    }
    if (r == KDA_OK)
        r = bwd_launch_all(q, k, v, gb, beta, scale, A_log, dtbb, lower_bound, cu_seqlens, num_seqs,
                           initial_state, initial_state_dtype, d_out, d_final_state, dq, dk, dv,
                           nullptr, dbeta, dA_log, ddtb, d_initial_state, B, T, H, K, stream,
                           (uint16_t *)dg);
    if (r == KDA_OK && ddtb) {
        hipLaunchKernelGGL(dtb_reduce_kernel, dim3((unsigned)((H + 255) / 256)), dim3(256), 0, s,
                           ddtb, H, K, ddt_bias);
        if (hipGetLastError() != hipSuccess) r = KDA_ERR_LAUNCH;
    }
    if (buf && hipFreeAsync(buf, s) != hipSuccess) r = KDA_ERR_LAUNCH;
    return r;
}

}  // extern "C"

namespace {

// Workspace of kda_fwd_noalloc: a file-scope device array.  Each device the
// library runs on holds its own copy until the process ends; its address on
// a device is read once with hipGetSymbolAddress (the array's name in host
// code is only a stand-in) and kept per device.  The last 256 bytes hold the
// optional cu_seqlens check's flag.
constexpr size_t kNoallocScratchBytes = KDA_NOALLOC_WORKSPACE_BYTES + 256;
__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

kda_status_t scratch_on_device(void **p) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return KDA_ERR_LAUNCH;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *p = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_fwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, float scale,
                             const float *A_log, const float *dt_bias, float lower_bound,
                             const int32_t *cu_seqlens, int32_t num_seqs,
                             const void *initial_state, kda_dtype_t initial_state_dtype,
                             void *final_state, kda_dtype_t final_state_dtype,
                             void *out,
                             int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                             void *stream)
{
    kda_status_t st = fwd_validate(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
                                   cu_seqlens, num_seqs, initial_state, initial_state_dtype,
                                   final_state, final_state_dtype, out, B, T, H, K, V, false);
    if (st != KDA_OK) return st;
    if (kda_workspace_size_hd(B, T, H, num_seqs, K) > KDA_NOALLOC_WORKSPACE_BYTES)
        return KDA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    void *ws = nullptr;
    if ((st = scratch_on_device(&ws)) != KDA_OK) return st;
    if (cu_seqlens && cu_check_enabled() &&
        (st = check_cu_flag(cu_seqlens, num_seqs, (int)((int64_t)B * T), s,
                            (int *)((uint8_t *)ws + KDA_NOALLOC_WORKSPACE_BYTES))) != KDA_OK)
        return st;
    const hipError_t e = fwd_launch(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound,
                                    cu_seqlens, num_seqs, initial_state, initial_state_dtype,
                                    final_state, final_state_dtype, out, B, T, H, K, V, s, false,
                                    ws);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_set_bwd_stage_events(void *const *events) {
    for (int i = 0; i < 6; ++i) t_bwd_events[i] = events ? (hipEvent_t)events[i] : nullptr;
    return KDA_OK;
}

kda_status_t kda_set_stage_events(void *before_intra, void *before_scan, void *after_scan) {
    t_stage_events[0] = (hipEvent_t)before_intra;
    t_stage_events[1] = (hipEvent_t)before_scan;
    t_stage_events[2] = (hipEvent_t)after_scan;
    return KDA_OK;
}

}  // extern "C"
