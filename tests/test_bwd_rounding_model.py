"""CPU model of the backward's storage roundings (no GPU).

The GPU backward keeps the chunk start states S0, the state gradients dS1,
the chunk inputs X = V - Kt S0 and their gradients dX in bf16 between its
kernels, and its two scans read bf16 records (Kt and Wm in the states
recurrence; Wm, scale Qt, Kt and scale M^T in the gradient recurrence).
This file restates the chunkwise backward of the chunk form ("Moonshot AI
Open-Sources FlashKDA", section "Why KDA?"; 16-token chunks) in fp64, with
those quantities optionally rounded to bf16, and checks:

  * without rounding it reproduces the fp64 gradient oracle's dA_log (so the
    restatement is the same derivative the oracle computes);
  * with the design's roundings, dA_log on the ragged K = V = 256 case of
    tests/test_bwd_gpu.py is off by more than the 5e-3 bar of the other
    gradients (about 1.9e-2), while the same inputs at K = V = 128 stay well
    inside it.  dA_log sums the log-decay gradient times the log-decay over
    every (token, channel); at 256 those terms cancel by a factor of about
    200.  This is why that GPU test holds dA_log to 3e-2 at K = 256.
"""
from __future__ import annotations

import numpy as np
import torch

import kda_inputs
import oracle
from formulations import _gate

CS = 16
RAGGED = dict(B=1, T=200, H=2, seq_lens=(0, 17, 1, 100, 82), initial_state=True)


def bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def chunkwise_dA_log(inp, d_out, d_final, K, lens, stored_bf16, records_bf16):
    """dA_log [H] by the chunkwise backward, per sequence and head."""
    f = lambda x: x.to(torch.float64).numpy()
    H = inp["q"].shape[2]
    scale, lb = inp["scale"], inp["lower_bound"]
    starts = np.concatenate([[0], np.cumsum(lens)])
    St = bf16 if stored_bf16 else (lambda x: x)
    Rc = bf16 if records_bf16 else (lambda x: x)
    out = np.zeros(H)
    for h in range(H):
        dtb = f(inp["dt_bias"]).reshape(H, K)[h]
        Al = float(inp["A_log"][h])
        for n in range(len(lens)):
            s0, s1 = starts[n], starts[n + 1]
            if s1 == s0:
                continue
            q, k, v, g = (f(inp[x][0, s0:s1, h]) for x in ("q", "k", "v", "g"))
            beta = 1.0 / (1.0 + np.exp(-f(inp["beta"][0, s0:s1, h])))
            a = _gate(g, dtb, Al, lb)
            S = f(inp["initial_state"][n, h])
            dO, dS = f(d_out[0, s0:s1, h]), f(d_final[n, h])
            L = s1 - s0
            ch = []
            for c in range(0, L, CS):
                sl = slice(c, min(L, c + CS))
                e = np.exp(np.cumsum(a[sl], axis=0))
                Kt, Qt, Kb = k[sl] * e, q[sl] * e, k[sl] / e
                m = e.shape[0]
                A = np.tril(Kt @ Kb.T, -1)
                Aqk = np.tril(Qt @ Kb.T)
                T = np.linalg.inv(np.eye(m) + beta[sl, None] * A)
                P = T * beta[sl][None, :]
                gam = e[-1]
                Wm = P.T @ Kb * gam[None, :]
                X = v[sl] - Rc(Kt) @ S
                ch.append(dict(sl=sl, Kt=Kt, Qt=Qt, Kb=Kb, Aqk=Aqk, T=T, P=P, M=Aqk @ P,
                               gam=gam, Wm=Wm, X=X, S0=S.copy()))
                S = gam[:, None] * S + Rc(Wm).T @ X
            for F in reversed(ch):
                F["dS1"] = dS.copy()
                dX = Rc(scale * F["M"].T) @ dO[F["sl"]] + Rc(F["Wm"]) @ St(dS)
                F["dX"] = dX
                dS = (F["gam"][:, None] * dS + Rc(scale * F["Qt"]).T @ dO[F["sl"]]
                      - Rc(F["Kt"]).T @ St(dX))
            for F in ch:
                sl = F["sl"]
                S0, dS1, X, dX = St(F["S0"]), St(F["dS1"]), St(F["X"]), St(F["dX"])
                dOc = dO[sl]
                dQt = scale * dOc @ S0.T
                dKt = -dX @ S0.T
                dWm = X @ dS1.T
                dM = scale * dOc @ X.T
                dAqk = np.tril(dM @ F["P"].T)
                dP = F["Aqk"].T @ dM + (F["Kb"] * F["gam"]) @ dWm.T
                dT = dP * beta[sl][None, :]
                dA = beta[sl][:, None] * np.tril(-F["T"].T @ dT @ F["T"].T, -1)
                dKbG = F["P"] @ dWm
                dKb = dAqk.T @ F["Qt"] + dA.T @ F["Kt"] + F["gam"] * dKbG
                dG = ((dKt + dA @ F["Kb"]) * F["Kt"] + (dQt + dAqk @ F["Kb"]) * F["Qt"]
                      - dKb * F["Kb"])
                gdg = F["gam"] * (np.sum(dS1 * S0, axis=1) + np.sum(dKbG * F["Kb"], axis=0))
                acc = gdg[None, :] + np.cumsum(dG[::-1], axis=0)[::-1]
                x = g[sl] + dtb
                y = -np.exp(Al) * (np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0.0))
                out[h] += np.sum(np.where(y >= lb, acc, 0.0) * y)
    return out


def ragged_case(K):
    kw = RAGGED
    inp = kda_inputs.random_small(910 + kw["T"] + kw["H"], K=K, V=K, **kw)
    d_out, d_final = kda_inputs.output_grads(911 + kw["T"], kw["B"], kw["T"], kw["H"], V=K,
                                             N=len(kw["seq_lens"]), K=K)
    return inp, d_out, d_final, oracle.numpy_backward(inp, d_out, d_final)["dA_log"]


def rel(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def test_exact_restatement_matches_the_oracle():
    inp, d_out, d_final, ref = ragged_case(256)
    got = chunkwise_dA_log(inp, d_out, d_final, 256, RAGGED["seq_lens"], False, False)
    assert rel(got, ref) < 1e-10


def test_bf16_storage_explains_the_dA_log_bar_at_256():
    inp, d_out, d_final, ref = ragged_case(256)
    lens = RAGGED["seq_lens"]
    stored = rel(chunkwise_dA_log(inp, d_out, d_final, 256, lens, True, False), ref)
    both = rel(chunkwise_dA_log(inp, d_out, d_final, 256, lens, True, True), ref)
    assert 5e-3 < stored < both < 3e-2, (stored, both)
    inp, d_out, d_final, ref = ragged_case(128)
    both128 = rel(chunkwise_dA_log(inp, d_out, d_final, 128, lens, True, True), ref)
    assert both128 < 5e-3, both128
