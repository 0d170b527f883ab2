"""Stage parity of the intra-chunk kernel: its hand-off records (decoded from
the documented register layouts) against fp64 chunk maths.

Per 16-token chunk with in-chunk inclusive cumulative log-decay G:
  gamma = e^{G_last}; Kt = k e^G; Qt = q e^G; Kb = k e^-G;
  Tb = (I + diag(beta) strict_lower(Kt Kb^T))^-1 diag(beta);
  Aqk = lower_incl(Qt Kb^T); M = Aqk Tb; W = Tb^T Kb diag(gamma).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
import oracle
from gpu_util import np64, to_device

pytestmark = pytest.mark.gpu

REC = 13312
CS = 16


def state_chan(t, rho):
    return 32 * (t // 2) + 8 * (rho // 4) + 4 * (t % 2) + rho % 4


def bf16_words_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode(rec: np.ndarray):
    """One 13312-byte record -> natural-layout matrices."""
    u16 = rec[:12800].view(np.uint16)
    Kt = np.zeros((CS, 128)); Qt = np.zeros((CS, 128)); W = np.zeros((CS, 128))
    kt = bf16_words_to_f64(u16[0:2048]).reshape(4, 64, 8)
    qt = bf16_words_to_f64(u16[2048:4096]).reshape(4, 64, 8)
    wt = bf16_words_to_f64(u16[4096:6144]).reshape(4, 64, 8)
    mm = bf16_words_to_f64(u16[6144:6400]).reshape(64, 4)
    for kb in range(4):
        for l in range(64):
            r, grp = l % 16, l // 16
            Kt[r, 32 * kb + 8 * grp: 32 * kb + 8 * grp + 8] = kt[kb, l]
            Qt[r, 32 * kb + 8 * grp: 32 * kb + 8 * grp + 8] = qt[kb, l]
    for tp in range(4):
        for m in range(64):
            rho, grp = m % 16, m // 16
            for half in range(2):
                ch = state_chan(2 * tp + half, rho)
                W[4 * grp: 4 * grp + 4, ch] = wt[tp, m, 4 * half: 4 * half + 4]
    M = np.zeros((CS, CS))
    for l in range(64):
        r, grp = l % 16, l // 16
        M[r, 4 * grp: 4 * grp + 4] = mm[l]
    gam = rec[12800:13312].view(np.float32).astype(np.float64)
    return Kt, Qt, W, M, gam


def expected_chunk(inp, t0, n_tok, h):
    f = lambda x: x.to(torch.float64).numpy()
    q = f(inp["q"][0, t0:t0 + n_tok, h]); k = f(inp["k"][0, t0:t0 + n_tok, h])
    g = f(inp["g"][0, t0:t0 + n_tok, h:h + 1])                   # [n, 1, K]
    H = inp["q"].shape[2]
    dtb = f(inp["dt_bias"]).reshape(H, 128)[h:h + 1]
    a = oracle.gate_log_decay(g, dtb.reshape(-1), f(inp["A_log"])[h:h + 1],
                              inp["lower_bound"])[:, 0]          # [n, K]
    beta = oracle.sigmoid(f(inp["beta"][0, t0:t0 + n_tok, h]))
    G = np.cumsum(a, axis=0)
    Kt = k * np.exp(G); Qt = q * np.exp(G); Kb = k * np.exp(-G)
    A = Kt @ Kb.T
    L = beta[:, None] * np.tril(A, -1)
    T = np.linalg.inv(np.eye(n_tok) + L)
    Tb = T * beta[None, :]
    Aq = np.tril(Qt @ Kb.T)
    return Kt, Qt, (Tb.T @ Kb) * np.exp(G[-1])[None, :], Aq @ Tb, np.exp(G[-1])


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("T", [64, 45])
def test_intra_stage_records(T):
    H = 3
    inp = kda_inputs.random_small(40 + T, B=1, T=T, H=H)
    d = to_device(inp)
    ws = kda.debug_intra(d["q"], d["k"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                         d["lower_bound"])
    torch.cuda.synchronize()
    recs = ws.cpu().numpy().reshape(-1, H, REC)
    for c in range((T + CS - 1) // CS):
        t0 = c * CS
        n_tok = min(CS, T - t0)
        for h in range(H):
            Kt, Qt, W, M, gam = decode(recs[c, h])
            eKt, eQt, eW, eM, egam = expected_chunk(inp, t0, n_tok, h)
            # gate + cumulative decay: fp32 exp2 of an fp32 sum
            assert np.all(np.abs(np.log(gam) - np.log(egam)) < 2e-4), (c, h)
            # decayed operands: one bf16 rounding (2^-8 relative bound) on top of fp32 maths
            for name, x, e in (("Kt", Kt, eKt), ("Qt", Qt, eQt)):
                assert np.all(np.abs(x[:n_tok] - e) <= 2.0 ** -8 * np.abs(e) + 1e-30), (name, c, h)
                assert np.all(x[n_tok:] == 0), (name, "padding rows", c, h)
            # M and W: fp32-accurate products rounded to bf16 once
            assert rel(W[:n_tok], eW) < 3e-3, (c, h, rel(W[:n_tok], eW))
            assert rel(M[:n_tok, :n_tok], eM) < 3e-3, (c, h, rel(M[:n_tok, :n_tok], eM))
            assert np.all(W[n_tok:] == 0) and np.all(M[n_tok:] == 0) and np.all(M[:, n_tok:] == 0)
