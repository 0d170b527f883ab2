"""Stage parity of the gate alone, through kda_debug_gate.

The gate stage evaluates, per token t, head h and key channel c, the
channel-wise log-decay a = max(-exp(A_log[h]) softplus(g + dt_bias), lb)
and beta = sigmoid(logit) ("Moonshot AI Rilis FlashKDA", API paragraphs;
"Moonshot AI Open-Sources FlashKDA", section "Why KDA?"), in base 2, and
the inclusive cumulative sum G of log2(e) a over the tokens of t's
16-token chunk (chunks start at each sequence's start).  kda_debug_gate
runs the intra stage's own gate code and returns G and beta in fp32; they
are compared element by element with the oracle's gate_log_decay and
sigmoid (pinned by the CPU tests) summed per chunk in fp64.

Error bound (fp32 on the GPU against fp64): each token's log2-decay is
exp2, an add, log2 and a multiply of fp32 values with x2 = (g + dt_bias)
log2 e, so its error is a few fp32 ulps of |la| plus A times a few ulps of
|x2| + 2 (log2(1 + 2^x2) changes by at most |dx2| for a change dx2 of x2,
and rounding 1 + 2^x2 costs an ulp of 1); the chunk sum adds an ulp of the
partial sum per token.  The test allows 2^-20 (sixteen ulps) of the sum
over the chunk's tokens up to t of |la| + A (|x2| + 2); beta likewise
2^-20 (1 + |logit|) relative.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
import oracle
from gpu_util import to_device

pytestmark = pytest.mark.gpu

CS = 16
LOG2E = 1.0 / math.log(2.0)
ULPS = 2.0 ** -20


def chunk_cumsum(x, starts):
    """Inclusive cumulative sum over axis 0 within 16-token chunks, chunks
    starting at each sequence start (starts: token offsets, last = T)."""
    out = np.empty_like(x)
    for s0, s1 in zip(starts[:-1], starts[1:]):
        for c in range(s0, s1, CS):
            e = min(s1, c + CS)
            out[c:e] = np.cumsum(x[c:e], axis=0)
    return out


def reference(inp, row):
    """(G, bound, beta, beta bound) of batch row `row` in fp64 from the
    oracle's gate, [T, H, K] and [T, H]."""
    f = lambda t: t.to(torch.float64).numpy()
    g = f(inp["g"][row])
    H, K = g.shape[-2], g.shape[-1]
    dtb = None if inp.get("dt_bias") is None else f(inp["dt_bias"])
    A_log = f(inp["A_log"])
    la = oracle.gate_log_decay(g, dtb, A_log, inp["lower_bound"]) * LOG2E
    A = np.exp(A_log).reshape(1, H, 1)
    x2 = (g if dtb is None else g + dtb.reshape(H, K)) * LOG2E
    T = g.shape[0]
    cu = inp.get("cu_seqlens")
    starts = [0, T] if cu is None else [int(v) for v in cu]
    G = chunk_cumsum(la, starts)
    bound = ULPS * chunk_cumsum(np.abs(la) + A * (np.abs(x2) + 2.0), starts)
    logit = f(inp["beta"][row])
    return G, bound, oracle.sigmoid(logit), ULPS * (1.0 + np.abs(logit))


def run_gate(inp):
    d = to_device(inp)
    G, b = kda.debug_gate(d["g"], d["beta"], d["A_log"], d.get("dt_bias"), d["lower_bound"],
                          cu_seqlens=d.get("cu_seqlens"))
    torch.cuda.synchronize()
    return G.cpu().double().numpy(), b.cpu().double().numpy()


def check(inp, tag):
    G, b = run_gate(inp)
    assert np.isfinite(G).all() and np.isfinite(b).all(), f"{tag}: unwritten elements"
    for row in range(G.shape[0]):
        Gr, bound, br, bbound = reference(inp, row)
        err = np.abs(G[row] - Gr)
        assert (err <= bound).all(), (tag, row, float(err.max()), float((err / bound).max()))
        berr = np.abs(b[row] - br)
        assert (berr <= bbound * br + 1e-30).all(), (tag, row, float(berr.max()))
    return G, b


@pytest.mark.parametrize("K", [64, 128, 256])
def test_ragged_varlen(K):
    """Several chunks per sequence, ragged tails, an empty and a one-token
    sequence."""
    inp = kda_inputs.random_small(300 + K, B=1, T=200, H=3, K=K, V=K, seq_lens=(0, 17, 1, 100, 82))
    check(inp, f"K={K}")


def test_batch_rows_without_cu_seqlens():
    inp = kda_inputs.random_small(311, B=3, T=40, H=2)
    check(inp, "B=3")


def test_no_dt_bias_and_poison():
    """dt_bias absent (zeros); the outputs start as NaN, so every token's
    entries must be written."""
    inp = kda_inputs.random_small(312, B=1, T=37, H=2)
    inp["dt_bias"] = None
    check(inp, "no dt_bias")


def test_no_decay_and_clamped_decay():
    """A_log = -inf: A = 0 and G = 0 exactly.  A gate far below the lower
    bound on every channel: each token's log2-decay is the bound, so G of
    the r-th token of a chunk is (r + 1) lb log2 e."""
    inp = kda_inputs.random_small(313, B=1, T=50, H=2)
    inp["A_log"] = torch.full_like(inp["A_log"], float("-inf"))
    G, _ = check(inp, "A = 0")
    assert (G == 0).all()
    inp = kda_inputs.random_small(314, B=1, T=50, H=2, lower_bound=kda.lower_bound_min())
    inp["A_log"] = torch.full_like(inp["A_log"], 4.0)
    inp["g"] = torch.full_like(inp["g"], 20.0)
    G, _ = check(inp, "clamped")
    lb2 = np.float32(kda.lower_bound_min() * LOG2E)
    r = (np.arange(50) % CS + 1).reshape(50, 1, 1)
    assert np.allclose(G[0], r * float(lb2), rtol=1e-6, atol=0)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["fixed_T8192_H96", "varlen_mixed12_H64"])
def test_full_size(name):
    """Every element of a full-size workload."""
    inp = kda_inputs.generate(kda_inputs.WORKLOADS[name])
    check(inp, name)
