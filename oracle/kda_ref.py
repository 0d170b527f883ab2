"""Plain fp64 CPU oracle for the Kimi Delta Attention (KDA) forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
do. It shares no code with the HIP library.

What it computes, written out token by token with no chunking, blocking or
re-association:

  * gate (log-decay, natural log): the pages name the gate's inputs (the
    pre-activation gate g and the fp32 parameters A_log, dt_bias and
    lower_bound; "Moonshot AI Rilis FlashKDA", API paragraphs) but not its
    formula. Reading taken here:
        a_t[c] = max(-exp(A_log[h]) * softplus(g_t[c] + dt_bias[h*K + c]),
                     lower_bound)
    so alpha_t = exp(a_t) lies in [exp(lower_bound), 1] per channel
    (channel-wise gating: same article, and "Moonshot AI Open-Sources
    FlashKDA", section "Why KDA?").
  * beta_t = sigmoid(beta logit): the kernel applies the sigmoid itself
    ("Moonshot AI Rilis FlashKDA", API paragraphs).
  * delta-rule state update with channel-wise decay applied first
    (a refinement of Gated DeltaNet: "Why KDA?"; gating plus delta update
    rule: productcool FAQ 1):
        S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
  * output from the updated state: o_t = scale * S_t^T q_t.
  * optional initial state per sequence (zeros when absent) and the final
    state per sequence; variable-length batches via cu_seqlens, the state
    resetting at each sequence start ("Moonshot AI Rilis FlashKDA", API and
    cu_seqlens paragraphs; productcool "Main Features" 3).

Every input arrives as the exact fp64 value of its bf16 / fp32 original.
"""
from __future__ import annotations

import numpy as np


def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + exp(x)) without overflow (numpy's logaddexp with 0)."""
    return np.logaddexp(0.0, x)


def sigmoid(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def gate_log_decay(g: np.ndarray, dt_bias: np.ndarray, A_log: np.ndarray,
                   lower_bound: float) -> np.ndarray:
    """Natural-log decay a = max(-exp(A_log[h]) * softplus(g + dt_bias), lb).

    g: [..., H, K]; dt_bias: [H*K] (or None for zeros); A_log: [H].
    """
    H, K = g.shape[-2], g.shape[-1]
    x = g if dt_bias is None else g + np.asarray(dt_bias, dtype=np.float64).reshape(H, K)
    A = np.exp(np.asarray(A_log, dtype=np.float64)).reshape(H, 1)
    with np.errstate(invalid="ignore"):
        a = -A * softplus(x)
    return np.maximum(a, lower_bound)


def _sequences(B: int, T: int, cu_seqlens):
    """(batch row, start, end) of every sequence, in order."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def kda_forward(q, k, v, g, beta, A_log, dt_bias, lower_bound, scale,
                initial_state=None, cu_seqlens=None):
    """Token-by-token fp64 KDA forward.

    q, k, g: [B, T, H, K]; v: [B, T, H, V]; beta: [B, T, H] (logits);
    A_log: [H]; dt_bias: [H*K] or None; initial_state: [N, H, K, V] or None;
    cu_seqlens: [N+1] offsets into T (then B == 1) or None.
    Returns (o [B, T, H, V], final_state [N, H, K, V]) in fp64.
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    seqs = _sequences(B, T, cu_seqlens)
    if cu_seqlens is not None and B != 1:
        raise ValueError("cu_seqlens requires B == 1")
    a = gate_log_decay(g, dt_bias, A_log, lower_bound)      # [B, T, H, K]
    alpha = np.exp(a)
    b = sigmoid(beta)                                        # [B, T, H]
    o = np.zeros((B, T, H, V), dtype=np.float64)
    final = np.zeros((len(seqs), H, K, V), dtype=np.float64)
    for n, (row, start, end) in enumerate(seqs):
        if initial_state is None:
            S = np.zeros((H, K, V), dtype=np.float64)
        else:
            S = np.array(initial_state[n], dtype=np.float64)   # [H, K, V]
        for t in range(start, end):
            kt = k[row, t]                                  # [H, K]
            # Diag(alpha_t) S_{t-1}
            S = alpha[row, t][:, :, None] * S
            # S <- S + beta k (v - S^T k)^T   ==  (I - beta k k^T) S + beta k v^T
            stk = np.einsum("hk,hkv->hv", kt, S)
            u = b[row, t][:, None] * (v[row, t] - stk)
            S = S + kt[:, :, None] * u[:, None, :]
            # o_t = scale * S_t^T q_t
            o[row, t] = scale * np.einsum("hk,hkv->hv", q[row, t], S)
        final[n] = S
    return o, final
