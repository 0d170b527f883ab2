/*
 * libkda — Kimi Delta Attention (KDA) chunked forward (prefill) for AMD
 * MI355X (gfx950).
 *
 * Operation (per sequence n, head h; state S is K x V, K = V = 64, 128 or 256):
 *
 *   a_t[c]  = max(-exp(A_log[h]) * softplus(g_t[c] + dt_bias[h*K + c]),
 *                 lower_bound)                      (log-decay, natural log)
 *   beta_t  = sigmoid(beta_logit_t)
 *   S_t     = (I - beta_t k_t k_t^T) Diag(exp(a_t)) S_{t-1} + beta_t k_t v_t^T
 *   o_t     = scale * S_t^T q_t
 *
 * The argument list follows the flash_kda.fwd call described in "Moonshot AI
 * Rilis FlashKDA" (API paragraphs): q, k, v, g (gate before activation) and
 * beta logits in bf16, an fp32 scale, a caller-allocated bf16 output, fp32
 * gate parameters A_log / dt_bias / lower_bound, optional initial and final
 * recurrent states in bf16 or fp32, and cu_seqlens for variable-length
 * batches.  The pages name the gate parameters but not the gate formula; the
 * clamped softplus form above is the reading this library implements.  The
 * original supports only K = V = 128 ("Moonshot AI Open-Sources FlashKDA",
 * section "Limitations before you integrate"); this library also takes
 * K = V = 64 and K = V = 256 in kda_fwd, kda_fwd_scalar_gate and kda_decode.  The
 * original ships only the forward pass (same section); kda_bwd here adds
 * the gradients (K = V = 64, 128 or 256).
 *
 * Conventions shared by every entry point:
 *   - Pointers are device pointers unless stated; every tensor is dense and
 *     row-major with the last dimension contiguous.  q, k, v, g, out and the
 *     state buffers must be 16-byte aligned; beta 2-byte; A_log, dt_bias and
 *     cu_seqlens 4-byte.
 *   - The caller owns every buffer.  The library never keeps a pointer past
 *     the call and never frees caller memory.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     legacy default stream of the current device).  Outputs are valid once
 *     the stream has completed the enqueued work.  No host synchronisation.
 *   - Host-side argument validation happens before any HIP call; nothing
 *     throws across the ABI.  Device-side contents (cu_seqlens values) are
 *     preconditions, not checked.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,   /* NULL/misaligned pointer, bad size or enum */
    KDA_ERR_UNSUPPORTED = 2,   /* valid but outside what the kernels handle */
    KDA_ERR_LAUNCH = 3,        /* a HIP launch or runtime call failed */
    KDA_ERR_OUT_OF_MEMORY = 4  /* the stream-ordered workspace could not be allocated */
} kda_status_t;

typedef enum {
    KDA_DTYPE_BF16 = 0,
    KDA_DTYPE_FP32 = 1
} kda_dtype_t;

/*
 * kda_fwd — KDA forward over a batch of sequences.
 *
 * Layout:
 *   q, k, g     bf16 [B, T, H, K]
 *   v           bf16 [B, T, H, V]
 *   beta        bf16 [B, T, H]       logits; the sigmoid is applied inside
 *   out         bf16 [B, T, H, V]    caller-allocated; every row in
 *                                    [0, B*T) is written exactly once
 *   A_log       fp32 [H]             per-head decay scale (A = exp(A_log))
 *   dt_bias     fp32 [H*K]           per (head, channel), index h*K + c;
 *                                    NULL means zeros
 *   scale       host fp32, finite
 *   lower_bound host fp32: finite, <= 0 and >= kda_lower_bound_min()
 *   cu_seqlens  int32 [num_seqs + 1] prefix offsets into the packed token
 *               axis, or NULL.  Non-NULL requires B == 1; then sequence n is
 *               tokens [cu[n], cu[n+1]).  Preconditions, not checked by
 *               default: cu[0] = 0, non-decreasing, cu[num_seqs] = T.
 *               With KDA_CHECK_CU_SEQLENS=1 in the environment, a one-block
 *               device check runs first and the call synchronises with the
 *               stream; bad contents then return KDA_ERR_INVALID_ARG with
 *               nothing else launched (kda_bwd alike).  Zero-length
 *               sequences are allowed.  NULL means B sequences of T tokens.
 *   num_seqs    N: B when cu_seqlens is NULL, else len(cu_seqlens) - 1
 *   initial_state  [N, H, K, V] in initial_state_dtype, or NULL (= zeros)
 *   final_state    [N, H, K, V] in final_state_dtype, or NULL (not written);
 *                  when given, every slab is written (a zero-length sequence
 *                  gets its initial state)
 *   B, T, H, K, V  sizes; K = V = 128, K = V = 256 (sixteen state row
 *                  tiles per column slice, 26 KB hand-off records), or
 *                  K = V = 64 (four state row tiles, 7 KB records).  When
 *                  B*T == 0 the
 *                  token buffers (q, k, v, g, beta, out) may be NULL; the
 *                  call then only writes final_state (= initial state)
 *
 * The state of each sequence starts from initial_state (or zeros) and does
 * not leak across sequences.  Internally the call takes a stream-ordered
 * workspace of kda_workspace_size_hd(B, T, H, num_seqs, K) bytes from a
 * library-owned memory pool on the current device and returns it on the
 * same stream (see kda_trim_workspace for how much of it stays reserved).
 *
 * Returns KDA_OK, or KDA_ERR_INVALID_ARG / KDA_ERR_UNSUPPORTED before any
 * HIP call, KDA_ERR_OUT_OF_MEMORY, or KDA_ERR_LAUNCH.
 */
kda_status_t kda_fwd(const void *q, const void *k, const void *v, const void *g,
                     const void *beta, float scale,
                     const float *A_log, const float *dt_bias, float lower_bound,
                     const int32_t *cu_seqlens, int32_t num_seqs,
                     const void *initial_state, kda_dtype_t initial_state_dtype,
                     void *final_state, kda_dtype_t final_state_dtype,
                     void *out,
                     int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                     void *stream);

/*
 * kda_fwd_scalar_gate — the Gated DeltaNet special case of the same forward:
 * one gate value per (token, head), shared by all K channels.  KDA is
 * described as Gated DeltaNet refined with channel-wise gating ("Moonshot
 * AI Open-Sources FlashKDA", section "Why KDA?"); this entry point is the
 * coarser gate, read as the same gate formula with per-head inputs:
 *
 *   a_t = max(-exp(A_log[h]) * softplus(g_t + dt_bias[h]), lower_bound)
 *
 * for every channel, which equals kda_fwd on g and dt_bias broadcast over
 * the channels (and the results are bit-identical to that call).
 *
 * Layout and everything else as kda_fwd, except:
 *   g           bf16 [B, T, H]       one gate pre-activation per token and head
 *                                    (2-byte aligned)
 *   dt_bias     fp32 [H] or NULL (= zeros)
 */
kda_status_t kda_fwd_scalar_gate(const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, float scale,
                                 const float *A_log, const float *dt_bias, float lower_bound,
                                 const int32_t *cu_seqlens, int32_t num_seqs,
                                 const void *initial_state, kda_dtype_t initial_state_dtype,
                                 void *final_state, kda_dtype_t final_state_dtype,
                                 void *out,
                                 int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                 void *stream);

/*
 * kda_fwd_noalloc — kda_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Arguments, layouts, results and errors are those of kda_fwd
 * (the results are bitwise identical to kda_fwd's), except:
 *   - no allocation or free happens: the workspace is a file-scope device
 *     array of the library, KDA_NOALLOC_WORKSPACE_BYTES (64 MiB) plus 256
 *     bytes, which every device the library runs on holds until the
 *     process ends;
 *   - calls whose workspace, kda_workspace_size_hd(B, T, H, num_seqs, K),
 *     exceeds KDA_NOALLOC_WORKSPACE_BYTES return KDA_ERR_UNSUPPORTED before
 *     any HIP call (e.g. T = 8192 fits up to H = 9 at K = 128);
 *   - every call on a device shares that device's array, which keeps the
 *     last call's contents (every byte a call reads it has written first):
 *     calls that overlap on one device (on different streams, or from
 *     different host threads without ordering) race and must not be made.
 */
#define KDA_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
kda_status_t kda_fwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, float scale,
                             const float *A_log, const float *dt_bias, float lower_bound,
                             const int32_t *cu_seqlens, int32_t num_seqs,
                             const void *initial_state, kda_dtype_t initial_state_dtype,
                             void *final_state, kda_dtype_t final_state_dtype,
                             void *out,
                             int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                             void *stream);

/*
 * kda_decode — one decode step: a single new token per sequence applied to
 * the recurrent state in place (the step after a prefill; it consumes the
 * final_state kda_fwd wrote, same layout).  "FlashKDA" product page, Main
 * Features (recurrent state between prefill and decode); the update is the
 * token recurrence above for one token:
 *
 *   S = (I - beta k k^T) Diag(exp(a)) S + beta k v^T,   o = scale * S^T q
 *
 * Layout:
 *   q, k, g     bf16 [N, H, K]       the new token of each sequence
 *   v           bf16 [N, H, V]
 *   beta        bf16 [N, H]          logits; the sigmoid is applied inside
 *   out         bf16 [N, H, V]       caller-allocated, every row written
 *   A_log       fp32 [H];  dt_bias fp32 [H*K] or NULL (= zeros)
 *   scale       host fp32, finite
 *   lower_bound host fp32, finite and <= 0 (no chunk factorisation here, so
 *               no lower limit beyond finiteness)
 *   state       [N, H, K, V] in state_dtype (bf16 or fp32), read and
 *               overwritten with the updated state (bf16: round to nearest
 *               even); the arithmetic is fp32 either way
 *   N, H, K, V  sizes; N, H >= 1; K = V = 64, 128 or 256 (one workgroup
 *               of K*K/64 threads per (sequence, head))
 *
 * No workspace.  Returns KDA_OK, KDA_ERR_INVALID_ARG / KDA_ERR_UNSUPPORTED
 * before any HIP call, or KDA_ERR_LAUNCH.
 */
kda_status_t kda_decode(const void *q, const void *k, const void *v, const void *g,
                        const void *beta, float scale,
                        const float *A_log, const float *dt_bias, float lower_bound,
                        void *state, kda_dtype_t state_dtype, void *out,
                        int32_t N, int32_t H, int32_t K, int32_t V, void *stream);

/*
 * kda_bwd — the backward pass for training: gradients of the forward above
 * with respect to every input.  The pages provide the forward only and leave
 * training to another backend ("Moonshot AI Open-Sources FlashKDA", section
 * "Limitations before you integrate"); this is the exact derivative of the
 * forward kda_fwd computes, for the loss
 *
 *   L = <d_out, o> + <d_final_state, final_state>
 *
 * (no gradient flows through the clamped branch of the gate).
 *
 * Inputs (as kda_fwd; K = V = 64, 128 or 256, each on kernels as wide as
 * the head):
 *   q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, cu_seqlens,
 *   num_seqs, initial_state (+ dtype), B, T, H, K, V
 *   d_out          bf16 [B, T, H, V]   gradient reaching o
 *   d_final_state  fp32 [N, H, K, V] or NULL (= zeros)
 * Outputs (caller-allocated, fully written):
 *   dq, dk, dg     bf16 [B, T, H, K]
 *   dv             bf16 [B, T, H, V]
 *   dbeta          bf16 [B, T, H]       gradient of the beta logits
 *   dA_log         fp32 [H]
 *   ddt_bias       fp32 [H*K] or NULL (not written)
 *   d_initial_state fp32 [N, H, K, V] or NULL (not written)
 *
 * Products run on bf16 MFMAs with fp32 accumulation: the stored states and
 * the scans' records are bf16, and fp32 operands whose precision matters
 * enter as (hi, lo) bf16 pairs; elementwise work is fp32.  Every sum runs in
 * a fixed order, so the results are bitwise reproducible.  Device workspace
 * of about 91 KiB per (16-token chunk slot, head) at K = 128 (31 KiB at 64,
 * 308 KiB at 256) comes from the library's stream-ordered pool (the two scans' records; X of every chunk and the
 * start state or the state gradient of every other chunk, in bf16; dX is
 * read back from dv).  The reverse scan runs on a
 * second stream the library creates once per device (non-blocking, default
 * priority), forked from `stream` after the prep kernel and joined back
 * before the chunk kernel by events, so the call as a whole stays ordered on
 * `stream`.  Returns KDA_OK, KDA_ERR_INVALID_ARG / KDA_ERR_UNSUPPORTED
 * before any HIP call, KDA_ERR_OUT_OF_MEMORY, or KDA_ERR_LAUNCH.
 */
kda_status_t kda_bwd(const void *q, const void *k, const void *v, const void *g,
                     const void *beta, float scale,
                     const float *A_log, const float *dt_bias, float lower_bound,
                     const int32_t *cu_seqlens, int32_t num_seqs,
                     const void *initial_state, kda_dtype_t initial_state_dtype,
                     const void *d_out, const float *d_final_state,
                     void *dq, void *dk, void *dv, void *dg, void *dbeta,
                     float *dA_log, float *ddt_bias, float *d_initial_state,
                     int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, void *stream);

/*
 * kda_bwd_scalar_gate — the backward of kda_fwd_scalar_gate (the Gated
 * DeltaNet form: one gate value per token and head for all key channels,
 * "Moonshot AI Open-Sources FlashKDA", section "Why KDA?").  That forward is
 * the channel-wise one with every channel's gate input equal, so this runs
 * kda_bwd on the gate and dt_bias broadcast over the channels and returns
 * the gate's and dt_bias's gradients summed over them (fp32 sums of the
 * channel-wise bf16 gate gradients, in channel order).
 *
 * Arguments as kda_bwd except:
 *   g         bf16 [B, T, H]   one pre-activation gate value per token, head
 *   dt_bias   fp32 [H] or NULL
 *   dg        bf16 [B, T, H]   (output)
 *   ddt_bias  fp32 [H] or NULL (output)
 * It takes, besides kda_bwd's workspace, 4 B T H K bytes (the broadcast
 * gate and its channel-wise gradient) and 8 H K bytes from the same pool,
 * stream-ordered.  Errors as kda_bwd.
 */
kda_status_t kda_bwd_scalar_gate(const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, float scale,
                                 const float *A_log, const float *dt_bias, float lower_bound,
                                 const int32_t *cu_seqlens, int32_t num_seqs,
                                 const void *initial_state, kda_dtype_t initial_state_dtype,
                                 const void *d_out, const float *d_final_state,
                                 void *dq, void *dk, void *dv, void *dg, void *dbeta,
                                 float *dA_log, float *ddt_bias, float *d_initial_state,
                                 int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                 void *stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char *kda_status_string(kda_status_t status);

/*
 * Smallest lower_bound the kernels accept.  Within one 16-token chunk the
 * kernels factor exp(G_r - G_i) as exp(G_r) * exp(-G_i) with G the in-chunk
 * cumulative log-decay, so 16 * |lower_bound| must keep both factors inside
 * the fp32 / bf16 normal range.
 */
float kda_lower_bound_min(void);

/* Tokens per chunk of the chunkwise algorithm (16). */
int32_t kda_chunk_size(void);

/*
 * Workspace memory.  kda_fwd, kda_fwd_scalar_gate and kda_bwd take their
 * workspace from a memory pool the library owns, one per device, with
 * stream-ordered allocations (hipMallocFromPoolAsync / hipFreeAsync on the
 * call's stream).  Freed blocks stay reserved for later calls up to 1 GiB
 * per device; whatever is above that is returned to the device when a
 * stream or the device synchronises.  (A backward at T = 8192, H = 96 takes
 * about 7.8 GB, of which 1 GiB then stays reserved.)
 *
 * kda_trim_workspace — returns reserved but unused pool memory of the
 * current device until at most keep_bytes stay reserved (keep_bytes = 0:
 * everything not in use).  Blocks still in use by enqueued work are not
 * released; call it after synchronising the streams that used the library.
 * Returns KDA_OK (also when the pool was never created) or KDA_ERR_LAUNCH.
 *
 * kda_workspace_reserved — bytes the pool of the current device holds
 * reserved (in use or cached); 0 when the pool was never created.
 */
kda_status_t kda_trim_workspace(size_t keep_bytes);
size_t kda_workspace_reserved(void);

/*
 * Bytes of device workspace one kda_fwd (or kda_fwd_scalar_gate) call with
 * these sizes at head dimension K = V = 128 takes from the pool on the
 * current device: one hand-off record (13 KB) per (16-token chunk slot,
 * head), floor(B T / 16) + num_seqs slots.  0 on invalid sizes.
 */
size_t kda_workspace_size(int32_t B, int32_t T, int32_t H, int32_t num_seqs);

/*
 * The same for any supported head dimension K (64, 128 or 256): records of
 * 7 KB (K = 64), 13 KB (K = 128) or 26 KB (K = 256) per chunk slot and head.
 * 0 on invalid sizes or an unsupported K.
 */
size_t kda_workspace_size_hd(int32_t B, int32_t T, int32_t H, int32_t num_seqs, int32_t K);

/*
 * kda_debug_gate — test entry: runs only the gate and the in-chunk
 * cumulative decay, through the same device code as the intra-chunk stage.
 * For every token t of head h (chunks of 16 tokens from each sequence's
 * start, the last one partial), with x = g[t, h, c] + dt_bias[h K + c]:
 *   a = max(-exp(A_log[h]) softplus(x), lower_bound)          (natural log)
 *   G[t, h, c]  = log2(e) * sum of a over the tokens of t's chunk up to t
 *   beta_out[t, h] = sigmoid(beta[t, h])
 * (the channel-wise decay and beta activation of "Moonshot AI Rilis
 * FlashKDA", API paragraphs, and "Moonshot AI Open-Sources FlashKDA",
 * section "Why KDA?"; base 2 as in section "What makes the kernel fast").
 * g, beta, A_log, dt_bias, lower_bound, cu_seqlens, num_seqs, B, T, H, K
 * as kda_fwd (K = 64, 128 or 256).  G: device fp32 [B, T, H, K], 16-byte
 * aligned; beta_out: device fp32 [B, T, H].  Every token's entries are
 * written.  Asynchronous on `stream`; errors as kda_fwd.
 */
kda_status_t kda_debug_gate(const void *g, const void *beta,
                            const float *A_log, const float *dt_bias, float lower_bound,
                            const int32_t *cu_seqlens, int32_t num_seqs,
                            float *G, float *beta_out,
                            int32_t B, int32_t T, int32_t H, int32_t K, void *stream);

/*
 * kda_debug_intra — test entry: runs only the intra-chunk stage (gate,
 * in-chunk cumulative decay, A_kk / A_qk products, triangular inverse) and
 * writes the hand-off record of every (chunk slot, head) into the caller's
 * `workspace` (device, kda_record_workspace_size(B, T, H, num_seqs, K)
 * bytes, 16-byte aligned).  Arguments as kda_fwd.  Record layout (per
 * 16-token chunk slot and head: 7168, 13312 or 26624 bytes for K = 64, 128
 * or 256) is described in the library source; tests decode it to
 * compare each stage with fp64 maths.
 */
size_t kda_record_workspace_size(int32_t B, int32_t T, int32_t H, int32_t num_seqs, int32_t K);
kda_status_t kda_debug_intra(const void *q, const void *k, const void *g,
                             const void *beta,
                             const float *A_log, const float *dt_bias, float lower_bound,
                             const int32_t *cu_seqlens, int32_t num_seqs,
                             int32_t B, int32_t T, int32_t H, int32_t K,
                             void *workspace, void *stream);

/*
 * kda_debug_scan_step — test entry: runs only the inter-chunk scan of the
 * forward (K = V = 64, 128 or 256) over hand-off records the caller
 * provides, one chunk step per record in order from the given state: per
 * chunk with state S (rows = key channels, columns = value channels)
 *   X = V - Kt S,   O = scale (Qt S + M X),   S <- diag(gamma) S + W^T X
 * (the chunkwise recurrence of the FlashKDA write-up, "Moonshot AI
 * Open-Sources FlashKDA", section "Why KDA?"; Kt, Qt, W, M and gamma as in
 * the records).  With sequences of at most 16 tokens this is exactly one
 * step from initial_state.  `records`: device, laid out as kda_debug_intra
 * writes them (kda_record_workspace_size(B, T, H, num_seqs, K) bytes,
 * 16-byte aligned; read only).  `v`, `out`, `cu_seqlens`, the states and
 * their dtypes as in kda_fwd (a NULL initial_state is zero, a NULL
 * final_state is not written).  `part_cols`: columns of the state per scan
 * workgroup, 32, 64 or 128 (at most V), or 0 for the width kda_fwd picks;
 * otherwise KDA_ERR_INVALID_ARG.  Other errors as kda_fwd.  Enqueued on
 * `stream`; returns before the kernel runs.
 */
kda_status_t kda_debug_scan_step(const void *v, const void *records, const int32_t *cu_seqlens,
                                 int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
                                 int32_t V, float scale, const void *initial_state,
                                 kda_dtype_t initial_state_dtype, void *final_state,
                                 kda_dtype_t final_state_dtype, void *out, int32_t part_cols,
                                 void *stream);

/*
 * kda_set_stage_events — instrumentation for per-kernel timing.  When set
 * (non-NULL hipEvent_t handles created by the caller on the device the calls
 * run on), the next kda_fwd calls made from the calling thread record
 * `before_intra` before the intra-chunk kernel, `before_scan` between the
 * intra-chunk and scan kernels and `after_scan` after the scan, all on the
 * call's stream.  Pass three NULLs to stop.  The setting is per host thread;
 * the library does not own the events.  Always returns KDA_OK.
 */
kda_status_t kda_set_stage_events(void *before_intra, void *before_scan, void *after_scan);

/*
 * kda_set_bwd_stage_events — the same instrumentation for kda_bwd: `events`
 * is NULL (stop) or an array of six hipEvent_t handles, recorded on the
 * call's stream: before the prep kernel, before the two scans, after the
 * states scan, after both scans (the reverse scan runs beside the states
 * scan on a library-owned second stream and is joined here), after the
 * chunk kernel and after the reduce kernel.  Per host thread; the array is
 * read at this call and the events are not owned.  Always returns KDA_OK.
 */
kda_status_t kda_set_bwd_stage_events(void *const *events);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
