"""Stage parity of the inter-chunk scan alone, through kda_debug_scan_step.

Per 16-token chunk with incoming state S (key channels x value channels)
the scan computes X = V - Kt S, O = scale (Qt S + M X) and the new state
diag(gamma) S + W^T X ("Moonshot AI Open-Sources FlashKDA", section "Why
KDA?": the chunkwise form).  Two checks, each at every column-part width the
launch can pick (32, 64, 128 columns per workgroup; 32 and 64 at K = V = 64)
and at head dimensions 64, 128 and 256:

  * Records the test encodes itself (random bf16 operands, zero rows past
    the chunk's length as the intra stage writes them) against fp64 maths
    on the same operands: once with the kernel's documented rounding points
    (S and X enter the products as bf16, O is stored as bf16) to a tight
    bound, once exact to the parity bar.
  * One chunk end to end: kda_debug_intra, then kda_debug_scan_step from an
    fp32 state, against the dense one-block formula of tests/formulations.py
    (pinned to the oracle by the CPU tests) at full, ragged and one-token
    chunks.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
from formulations import dense_sequence
from gpu_util import MAX_ABS_TOL, REL_L2_TOL, to_device
from records import CS, REC, bf16_round, decode, encode


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


WIDTHS = [(128, 32), (128, 64), (128, 128), (64, 32), (64, 64), (256, 32), (256, 64), (256, 128)]
LENGTHS = [16, 9, 1]


def tile(D):
    """Key channels of the record tiles at head dimension D (the head
    dimension itself)."""
    return D


def test_record_codec_round_trip():
    """encode and decode are inverse on bf16-exact operands (CPU)."""
    rng = np.random.default_rng(0)
    for KT in (128, 256):
        Kt, Qt, W = (bf16_round(rng.normal(size=(CS, KT))) for _ in range(3))
        M = bf16_round(rng.normal(size=(CS, CS)))
        gam = rng.random(KT).astype(np.float32)
        out = decode(encode(Kt, Qt, W, M, gam, KT=KT), KT)
        for x, y in zip(out, (Kt, Qt, W, M, gam.astype(np.float64))):
            assert np.array_equal(x, y)


def chunk_operands(rng, H, D, n, exact):
    """Per head: Kt, Qt, W [16, KT] and M [16, 16] (rows, and M's columns,
    past n zero as the intra stage writes them; channels past D zero), gamma
    [KT] in (0.05, 1], S0 [D, D] and v [n, D] (KT = tile(D)).

    exact: quantised values whose products and partial sums are all exact in
    fp32 (Kt, Qt, W, M in {-2..2}/8, S0 in {0, +-1/8, +-1/4, +-1/2}, v in
    {-64..64}/16): P = Kt S0 and X = V - P are exact, X's bf16 rounding is
    the same on both sides, Qt S0 + M X is exact and the output is a scaled
    bf16 rounding of an exact value, so the kernel's output must match
    bitwise and its state to a few fp32 ulps (gamma S0 is exact too; only
    the final sum of the update rounds).  Otherwise: random normal values
    rounded to bf16."""
    ops = []
    KT = tile(D)
    for _ in range(H):
        Kt = np.zeros((CS, KT)); Qt = np.zeros((CS, KT)); W = np.zeros((CS, KT))
        M = np.zeros((CS, CS)); gam = np.zeros(KT)
        if exact:
            q8 = lambda shape: rng.integers(-2, 3, size=shape) / 8.0
            Kt[:n, :D], Qt[:n, :D], W[:n, :D] = q8((n, D)), q8((n, D)), q8((n, D))
            M[:n, :n] = np.tril(q8((n, n)))
            S0 = rng.choice(np.array([0.0, 0.125, -0.125, 0.25, -0.25, 0.5, -0.5]), size=(D, D))
            v = rng.integers(-64, 65, size=(n, D)) / 16.0
        else:
            b = lambda shape, s: bf16_round(rng.normal(scale=s, size=shape))
            Kt[:n, :D], Qt[:n, :D], W[:n, :D] = b((n, D), 0.1), b((n, D), 0.1), b((n, D), 0.1)
            M[:n, :n] = np.tril(b((n, n), 0.2))
            S0 = rng.normal(scale=0.5, size=(D, D)).astype(np.float32).astype(np.float64)
            v = b((n, D), 1.0)
        gam[:D] = rng.uniform(0.05, 1.0, size=D).astype(np.float32)
        ops.append((Kt, Qt, W, M, gam, S0, v))
    return ops


def run_scan_step(ops, D, n, scale, cw):
    H = len(ops)
    rec = np.stack([encode(*o[:5], KT=tile(D)) for o in ops])   # [H, bytes]: chunk slot 0
    need = int(kda.load().kda_record_workspace_size(1, n, H, 1, D))
    recs = torch.zeros(max(need, rec.size), dtype=torch.uint8)
    recs[:rec.size] = torch.from_numpy(rec.reshape(-1))
    v = torch.from_numpy(np.stack([o[6] for o in ops], axis=1)[None]).to(torch.bfloat16)
    S0 = torch.from_numpy(np.stack([o[5] for o in ops])[None]).float()
    out = torch.full((1, n, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((1, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    kda.debug_scan_step(v.cuda(), recs.cuda(), scale, out, initial_state=S0.cuda(), final_state=fin,
                        part_cols=cw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()[0].astype(np.float64), fin.cpu().numpy()[0].astype(np.float64)


@pytest.mark.gpu
@pytest.mark.parametrize("D,cw", WIDTHS)
@pytest.mark.parametrize("n", LENGTHS)
def test_scan_step_exact_operands(D, cw, n):
    """Quantised records: output bitwise, new state within 4 fp32 ulps of
    the magnitudes summed."""
    H, scale = 3, 0.125
    ops = chunk_operands(np.random.default_rng(1000 * D + 10 * cw + n), H, D, n, exact=True)
    o, S1 = run_scan_step(ops, D, n, scale, cw)
    for h, (Kt, Qt, W, M, gam, S0, v) in enumerate(ops):
        Kt, Qt, W, g = Kt[:n, :D], Qt[:n, :D], W[:, :D], gam[:D]
        X = np.zeros((CS, D))
        X[:n] = bf16_round(v - Kt @ S0)                      # exact difference, rounded once
        O = bf16_round(scale * (Qt @ S0 + (M @ X)[:n]))
        assert np.array_equal(o[:, h], O), (h, np.abs(o[:, h] - O).max())
        S_new = g[:, None] * S0 + W.T @ X
        mag = np.abs(g[:, None] * S0) + np.abs(W.T) @ np.abs(X)
        assert np.all(np.abs(S1[h] - S_new) <= 4 * 2.0 ** -24 * mag), (h, np.abs(S1[h] - S_new).max())


@pytest.mark.gpu
@pytest.mark.parametrize("D,cw", WIDTHS)
@pytest.mark.parametrize("n", LENGTHS)
def test_scan_step_random_operands(D, cw, n):
    """Random bf16 records against exact fp64 maths, to the parity bar."""
    H, scale = 3, D ** -0.5
    ops = chunk_operands(np.random.default_rng(7000 + 1000 * D + 10 * cw + n), H, D, n, exact=False)
    o, S1 = run_scan_step(ops, D, n, scale, cw)
    for h, (Kt, Qt, W, M, gam, S0, v) in enumerate(ops):
        Kt, Qt, W, g = Kt[:n, :D], Qt[:n, :D], W[:, :D], gam[:D]
        X = np.zeros((CS, D))
        X[:n] = v - Kt @ S0
        O = scale * (Qt @ S0 + (M @ X)[:n])
        S_new = g[:, None] * S0 + W.T @ X
        assert rel(o[:, h], O) < REL_L2_TOL and np.abs(o[:, h] - O).max() < MAX_ABS_TOL, (h, rel(o[:, h], O))
        assert rel(S1[h], S_new) < REL_L2_TOL and np.abs(S1[h] - S_new).max() < MAX_ABS_TOL, (h, rel(S1[h], S_new))


@pytest.mark.gpu
@pytest.mark.parametrize("D,cw", WIDTHS)
@pytest.mark.parametrize("n", LENGTHS)
def test_one_chunk_intra_then_scan_step(D, cw, n):
    """kda_debug_intra then kda_debug_scan_step on one chunk from an fp32
    state, against the dense one-block formula."""
    H = 3
    inp = kda_inputs.random_small(500 + n + cw + D, B=1, T=n, H=H, K=D, V=D)
    S0 = (torch.randn(1, H, D, D, generator=torch.Generator().manual_seed(7 + n)) * 0.3).float()
    d = to_device(inp)
    recs = kda.debug_intra(d["q"], d["k"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                           d["lower_bound"])
    out = torch.full((1, n, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((1, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    kda.debug_scan_step(d["v"], recs, inp["scale"], out, initial_state=S0.cuda(), final_state=fin,
                        part_cols=cw)
    torch.cuda.synchronize()
    f = lambda x: x.to(torch.float64).numpy()
    dtb = f(inp["dt_bias"]).reshape(H, D)
    for h in range(H):
        O, S_end = dense_sequence(f(inp["q"][0, :, h]), f(inp["k"][0, :, h]), f(inp["v"][0, :, h]),
                                  f(inp["g"][0, :, h]), f(inp["beta"][0, :, h]),
                                  float(inp["A_log"][h]), dtb[h], inp["lower_bound"], inp["scale"],
                                  f(S0[0, h]))
        o = f(out[0, :, h].cpu())
        s1 = f(fin[0, h].cpu())
        assert rel(o, O) < REL_L2_TOL and np.abs(o - O).max() < MAX_ABS_TOL, (h, rel(o, O))
        assert rel(s1, S_end) < REL_L2_TOL and np.abs(s1 - S_end).max() < MAX_ABS_TOL, (h, rel(s1, S_end))


@pytest.mark.gpu
def test_scan_step_rejects_bad_width():
    v = torch.zeros(1, 16, 2, 64, dtype=torch.bfloat16, device="cuda")
    recs = torch.zeros(REC * 2 * 2, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(v)
    for cw in (16, 128, 96):
        with pytest.raises(kda.KDAError):
            kda.debug_scan_step(v, recs, 0.125, out, part_cols=cw)
