"""Independent fp64 formulations used to pin the oracle (test helpers).

None of these calls the oracle's recurrence. They restate the method in
other, mathematically equivalent forms:

  * dense_sequence: the whole sequence as one block.  With G_r the inclusive
    cumulative log-decay and e_r = beta_r (v_r - (D_r S_{r-1})^T k_r), the
    recurrence unrolls to S_r = Gamma_r S0 + sum_{i<=r} Gamma_r Gamma_i^-1
    k_i e_i^T, so E solves the unit lower-triangular system
      (I + diag(beta) strict_lower(A)) E = diag(beta) (V - (K * e^G) S0),
      A[r, i] = sum_c k_r[c] k_i[c] exp(G_r[c] - G_i[c]),
    and o_r = scale ((q_r * e^{G_r}) S0 + sum_{i<=r} Bq[r, i] e_i) with
      Bq[r, i] = sum_c q_r[c] k_i[c] exp(G_r[c] - G_i[c]).
    A and Bq are built element by element (T x T x K tensor of decays) and the
    system is solved with numpy.linalg.solve: no factorisation of the decay.
    This is the "specialized DPLR" chunkwise form of "Moonshot AI
    Open-Sources FlashKDA", section "Why KDA?", with one chunk.
  * chunked_sequence: the same block formula applied chunk by chunk with the
    state carried between chunks (any chunk size, ragged last chunk).
  * matrix_recurrence: explicit K x K transition matrices
    M_t = (I - beta_t k_t k_t^T) Diag(alpha_t) for tiny K.
"""
from __future__ import annotations

import numpy as np


def _gate(g, dt_bias, A_log_h, lb):
    x = g + dt_bias
    sp = np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0.0)
    return np.maximum(-np.exp(A_log_h) * sp, lb)


def dense_block(q, k, v, a, beta, S0, scale):
    """One block: q,k [L,K], v [L,V], a [L,K] log-decay, beta [L] in (0,1)."""
    L, K = k.shape
    G = np.cumsum(a, axis=0)                                  # [L, K]
    r_idx = np.arange(L)[:, None]
    i_idx = np.arange(L)[None, :]
    causal = (i_idx <= r_idx)                                 # i <= r
    diff = G[:, None, :] - G[None, :, :]                      # [r, i, c]
    decay = np.where(causal[:, :, None], np.exp(np.where(causal[:, :, None], diff, 0.0)), 0.0)
    A = np.einsum("rc,ic,ric->ri", k, k, decay)
    Bq = np.einsum("rc,ic,ric->ri", q, k, decay)
    strict = (i_idx < r_idx)
    Lmat = beta[:, None] * np.where(strict, A, 0.0)
    Kg = k * np.exp(G)
    rhs = beta[:, None] * (v - Kg @ S0)
    E = np.linalg.solve(np.eye(L) + Lmat, rhs)
    O = scale * ((q * np.exp(G)) @ S0 + np.where(causal, Bq, 0.0) @ E)
    S_end = np.exp(G[-1])[:, None] * S0 + (k * np.exp(G[-1][None, :] - G)).T @ E
    return O, S_end


def dense_sequence(q, k, v, g, beta_logit, A_log_h, dt_bias_h, lb, scale, S0):
    a = _gate(g, dt_bias_h, A_log_h, lb)
    beta = 1.0 / (1.0 + np.exp(-beta_logit))
    return dense_block(q, k, v, a, beta, S0, scale)


def chunked_sequence(q, k, v, g, beta_logit, A_log_h, dt_bias_h, lb, scale, S0, chunk):
    a = _gate(g, dt_bias_h, A_log_h, lb)
    beta = 1.0 / (1.0 + np.exp(-beta_logit))
    L = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    outs = []
    for s in range(0, L, chunk):
        e = min(L, s + chunk)
        O, S = dense_block(q[s:e], k[s:e], v[s:e], a[s:e], beta[s:e], S, scale)
        outs.append(O)
    return np.concatenate(outs, axis=0) if outs else np.zeros((0, v.shape[1])), S


def matrix_recurrence(q, k, v, g, beta_logit, A_log_h, dt_bias_h, lb, scale, S0):
    a = _gate(g, dt_bias_h, A_log_h, lb)
    beta = 1.0 / (1.0 + np.exp(-beta_logit))
    K = k.shape[1]
    S = np.array(S0, dtype=np.float64)
    outs = []
    for t in range(q.shape[0]):
        M = (np.eye(K) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(a[t]))
        S = M @ S + beta[t] * np.outer(k[t], v[t])
        outs.append(scale * (S.T @ q[t]))
    return np.array(outs), S
