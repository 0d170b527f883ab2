// Host-side launchers of the libkda kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Intra-chunk stage over num_slots chunk slots x H heads; writes hand-off
// records (RecLayout<K>::BYTES each, slot-major then head) into ws.
// K = 64, 128 or 256, the width of the record's tiles.  scalar_gate: g is
// [B*T, H] and dt_bias [H] (one gate value per token and head).
hipError_t launch_intra(const uint16_t *q, const uint16_t *k, const uint16_t *g,
                        const uint16_t *beta, const float *A_log, const float *dt_bias,
                        float lower_bound, const int32_t *cu, int N, int T, int H, int K,
                        int64_t num_slots, uint8_t *ws, hipStream_t stream,
                        bool scalar_gate = false);

// The gate stage alone (a stage entry): G [B*T, H, K] fp32, the in-chunk
// inclusive cumulative base-2 log-decay of every token, and beta
// [B*T, H] fp32.  K = 64, 128 or 256.
hipError_t launch_gate(const uint16_t *g, const uint16_t *beta, const float *A_log,
                       const float *dt_bias, float lower_bound, const int32_t *cu, int N, int T,
                       int H, int K, int64_t num_slots, float *G_out, float *beta_out,
                       hipStream_t stream);

// Inter-chunk scan over N sequences x H heads.  K = V = 64, 128 or 256, the
// height of the state tiles.  part_cols: columns of the state per workgroup
// (32, 64 or 128, at most V); 0 = chosen from the number of (sequence,
// head) units and compute units.
hipError_t launch_scan(const uint16_t *v, const uint8_t *ws, const int32_t *cu, int N, int T,
                       int H, int K, int V, float scale, const void *init, int init_fp32,
                       void *fin, int fin_fp32, uint16_t *out, hipStream_t stream,
                       int part_cols = 0);

// Forward scan of the backward (K = V = 64, 128 or 256): the state from init
// (bf16 or fp32 [N, H, V, V], or NULL) through every chunk over the states
// records srec (StatesRecT<V>: Kt, Wm, the chunk decay); stores per (chunk
// slot, head) S0 of the even chunks (bf16, [part of 16 columns][V rows][16])
// and X (bf16 [16][V]).
hipError_t launch_bwd_fscan(const uint16_t *v, const uint8_t *srec, const int32_t *cu, int N, int T,
                            int H, int V, const void *init, int init_fp32, uint16_t *s0, uint16_t *xws,
                            hipStream_t stream);

// Reverse scan of the backward (K = V = 64, 128 or 256): the state gradient from
// dfin (fp32 [N, H, V, V] or NULL) back through every chunk, over the
// reverse records rrec (RecLayout<V>, per (chunk slot, head)); writes dv
// (= dX), dinit (fp32, if not NULL), and per (chunk slot, head) dS1 of the
// odd chunks and the last one (bf16, [part of 16 columns][V rows][16]).
hipError_t launch_bwd_rscan(const uint16_t *dout, const uint8_t *rrec, const int32_t *cu, int N,
                            int T, int H, int V, const float *dfin, float *dinit, uint16_t *dv,
                            uint16_t *ds1, hipStream_t stream);

// One-token decode step on N x H states of D x D (D = 64, 128 or 256) in
// place (fp32 or bf16).
hipError_t launch_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const uint16_t *g, const uint16_t *beta, float scale,
                         const float *A_log, const float *dt_bias, float lower_bound, int N,
                         int H, int D, void *state, int state_fp32, uint16_t *out,
                         hipStream_t stream);

// Backward pass (K = V = 64, 128 or 256, each on kernels as wide as the head):
// five launches on `stream` (one of them on a side stream, joined back)
// using the caller's workspace of bwd_workspace_bytes(num_slots, H, K) bytes
// (16-byte aligned).  events: NULL, or six events recorded before each
// launch and after the last.  dg_scalar: the Gated DeltaNet form (g and
// dt_bias broadcast over the channels by the caller): the gate gradient
// summed over the channels in fp32, written there as bf16 [B*T, H]; dg is
// then not written.
size_t bwd_workspace_bytes(int64_t num_slots, int H, int K);
hipError_t launch_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                      const uint16_t *beta, float scale, const float *A_log,
                      const float *dt_bias, float lower_bound, const int32_t *cu, int N, int T,
                      int H, int K, int64_t num_slots, const void *init, int init_fp32,
                      const uint16_t *dout, const float *dfin, uint16_t *dq, uint16_t *dk,
                      uint16_t *dv, uint16_t *dg, uint16_t *dbeta, float *dA_log,
                      float *ddt_bias, float *dinit, void *ws, hipStream_t stream,
                      const hipEvent_t *events, uint16_t *dg_scalar = nullptr);

}  // namespace kda
