"""Plain fp64 CPU oracle for the gradient of the KDA forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module; only the tests and the benchmark's CPU-baseline leg do. It shares no
code with the HIP library.

The pages ship the forward only and leave training to another backend
("Moonshot AI Open-Sources FlashKDA", section "Limitations before you
integrate"); the gradient has no definition of its own there.  What this
module computes is the exact derivative of the forward of kda_ref.kda_forward
(same gate, beta, state update and output), by reverse-mode differentiation
of the token recurrence, one token at a time, in the reverse of the forward's
order.  For the scalar loss

    L = <d_out, o> + <d_final, final_state>

it returns dL/d(every input).  Per token, with S' = Diag(alpha) S_prev,
w = S'^T k, u = beta (v - w), S = S' + k u^T and o = scale S^T q, the
adjoint step taking dS (the gradient reaching S) to the gradient reaching
S_prev is the chain rule through those five assignments, last first:

    dS      += scale q do^T                    dq      = scale S do
    dk       = dS u                            du      = dS^T k
    dbeta_s  = <du, v - w>                     dv      = beta du
    dw       = -beta du
    dS'      = dS + k dw^T                     dk     += S' dw
    dalpha   = rowsum(dS' * S_prev)            dS_prev = Diag(alpha) dS'

and through the gate a = max(y, lb), y = -exp(A_log) softplus(g + dt_bias),
alpha = exp(a), beta_s = sigmoid(logit):

    da = alpha dalpha;  dy = da where y >= lb, else 0
    dg = dy (-exp(A_log)) sigmoid(g + dt_bias);  ddt_bias = sum of dg over tokens
    dA_log = sum over tokens and channels of dy y
    dlogit = dbeta_s beta_s (1 - beta_s)

Reading taken at the clamp: where y equals lb exactly the gradient goes to y
(the clamped branch is the constant).  Forward states are recomputed from
checkpoints kept every `checkpoint` tokens, which changes no arithmetic.
"""
from __future__ import annotations

import numpy as np

from .kda_ref import _sequences, sigmoid, softplus


def kda_backward(q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, d_out,
                 d_final=None, initial_state=None, cu_seqlens=None, checkpoint=64):
    """Gradients of L = <d_out, o> + <d_final, final_state> (fp64).

    Shapes as kda_ref.kda_forward; d_out: [B, T, H, V]; d_final: [N, H, K, V]
    or None (zeros).  Returns a dict with dq, dk, dg [B, T, H, K], dv
    [B, T, H, V], dbeta [B, T, H], dA_log [H], ddt_bias [H*K] and
    d_initial_state [N, H, K, V].
    """
    f64 = lambda x: None if x is None else np.asarray(x, dtype=np.float64)
    q, k, v, g, beta, d_out = (f64(x) for x in (q, k, v, g, beta, d_out))
    d_final, initial_state = f64(d_final), f64(initial_state)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if cu_seqlens is not None and B != 1:
        raise ValueError("cu_seqlens requires B == 1")
    seqs = _sequences(B, T, cu_seqlens)

    # gate and beta (forward values)
    dtb = np.zeros((H, K)) if dt_bias is None else f64(dt_bias).reshape(H, K)
    x = g + dtb                                           # [B, T, H, K]
    A = np.exp(f64(A_log)).reshape(H, 1)
    y = -A * softplus(x)
    a = np.maximum(y, lower_bound)
    alpha = np.exp(a)
    b = sigmoid(beta)                                     # [B, T, H]

    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dalpha = np.zeros_like(q)
    db = np.zeros_like(b)
    d_init = np.zeros((len(seqs), H, K, V))

    def step(row, t, S_prev):
        """Forward token step; returns (S', w, u, S)."""
        Sp = alpha[row, t][:, :, None] * S_prev
        w = np.einsum("hk,hkv->hv", k[row, t], Sp)
        u = b[row, t][:, None] * (v[row, t] - w)
        S = Sp + k[row, t][:, :, None] * u[:, None, :]
        return Sp, w, u, S

    for n, (row, start, end) in enumerate(seqs):
        S = np.zeros((H, K, V)) if initial_state is None else initial_state[n].copy()
        # forward: states at the segment starts
        starts = list(range(start, end, checkpoint))
        saved = {}
        for t in range(start, end):
            if (t - start) % checkpoint == 0:
                saved[t] = S
            S = step(row, t, S)[3]
        dS = np.zeros((H, K, V)) if d_final is None else d_final[n].copy()
        for s0 in reversed(starts):
            s1 = min(s0 + checkpoint, end)
            prev = [saved[s0]]                            # state before each token of the segment
            for t in range(s0, s1 - 1):
                prev.append(step(row, t, prev[-1])[3])
            for t in range(s1 - 1, s0 - 1, -1):
                S_prev = prev[t - s0]
                Sp, w, u, S_t = step(row, t, S_prev)
                qt, kt, do = q[row, t], k[row, t], d_out[row, t]
                dS = dS + scale * qt[:, :, None] * do[:, None, :]
                dq[row, t] = scale * np.einsum("hkv,hv->hk", S_t, do)
                dk_t = np.einsum("hkv,hv->hk", dS, u)
                du = np.einsum("hkv,hk->hv", dS, kt)
                db[row, t] = np.sum(du * (v[row, t] - w), axis=-1)
                dv[row, t] = b[row, t][:, None] * du
                dw = -b[row, t][:, None] * du
                dSp = dS + kt[:, :, None] * dw[:, None, :]
                dk_t = dk_t + np.einsum("hkv,hv->hk", Sp, dw)
                dk[row, t] = dk_t
                dalpha[row, t] = np.sum(dSp * S_prev, axis=-1)
                dS = alpha[row, t][:, :, None] * dSp
        d_init[n] = dS

    da = alpha * dalpha
    dy = np.where(y >= lower_bound, da, 0.0)
    dx = dy * (-A) * sigmoid(x)
    dg = dx
    ddt_bias = dx.sum(axis=(0, 1)).reshape(H * K)
    dA_log = (dy * y).sum(axis=(0, 1, 3))
    dbeta = db * b * (1.0 - b)
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dA_log=dA_log,
                ddt_bias=ddt_bias, d_initial_state=d_init)
