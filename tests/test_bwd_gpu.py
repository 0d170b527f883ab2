"""GPU parity of the backward pass (kda_bwd through the C-ABI) against the
fp64 gradient oracle (oracle/kda_ref_bwd.py; at full size its C restatement,
oracle.cref_backward, on every head) on the same seeded inputs and incoming
gradients.

Bar, per gradient tensor: relative L2 error <= 5e-3 (the forward's bar) and
max-abs error <= 2e-2 x the largest reference magnitude.  The kernels compute
in fp32 and round dq, dk, dv, dg, dbeta to bf16 once (relative rounding
<= 2^-9 per element); the fp32 chunk products add errors of a few 1e-6
relative, so both bounds hold with a wide margin unless a term is wrong.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
import oracle
from gpu_util import to_device

pytestmark = pytest.mark.gpu

REL_L2 = 5e-3
MAX_REL = 2e-2
TOKEN_GRADS = ("dq", "dk", "dv", "dg", "dbeta")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    kda.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def run_bwd(d, d_out, d_final, want_dtb=True, want_dinit=True):
    q = d["q"]
    B, T, H, K = q.shape
    V = d["v"].shape[-1]
    cu = d.get("cu_seqlens")
    N = B if cu is None else cu.numel() - 1
    nan = float("nan")
    bf = torch.bfloat16
    o = dict(dq=torch.full_like(q, nan), dk=torch.full_like(q, nan), dg=torch.full_like(q, nan),
             dv=torch.full((B, T, H, V), nan, dtype=bf, device="cuda"),
             dbeta=torch.full((B, T, H), nan, dtype=bf, device="cuda"),
             dA_log=torch.full((H,), nan, device="cuda"))
    o["ddt_bias"] = torch.full((H * K,), nan, device="cuda") if want_dtb else None
    o["d_initial_state"] = torch.full((N, H, K, V), nan, device="cuda") if want_dinit else None
    kda.bwd(q, d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"], d.get("dt_bias"),
            d["lower_bound"], d_out.cuda(), o["dq"], o["dk"], o["dv"], o["dg"], o["dbeta"],
            o["dA_log"], ddt_bias=o["ddt_bias"], initial_state=d.get("initial_state"),
            d_final_state=None if d_final is None else d_final.cuda(),
            d_initial_state=o["d_initial_state"], cu_seqlens=cu)
    torch.cuda.synchronize()
    return o


def compare(name, got, ref, rel_l2=None):
    x = got.float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else got
    ref = np.asarray(ref, dtype=np.float64).reshape(x.shape)
    assert np.isfinite(x).all(), f"{name}: non-finite (unwritten) elements"
    scale = np.max(np.abs(ref))
    if scale == 0.0:
        assert np.max(np.abs(x)) == 0.0, name
        return 0.0
    rl2 = float(np.linalg.norm(x - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(x - ref)) / scale)
    print(f"{name}: rel_l2={rl2:.2e} max/scale={mx:.2e}", flush=True)
    bar = REL_L2 if rel_l2 is None else rel_l2
    assert rl2 <= bar and mx <= max(MAX_REL, bar), (name, rl2, mx)
    return rl2


def check(inp, out, d_out, d_final, alog_rel_l2=None, full=False):
    """Every gradient of every head against the oracle: the numpy one, or
    with full=True its C restatement (for the larger cases), each head's
    slice of the token gradients and the initial-state gradient then also
    held to the bar on its own, so that one wrong head cannot hide in a
    whole-tensor norm.  The per-head check covers slices of at least 4096
    elements: dbeta of a short sequence holds a few hundred values per head,
    and its bf16 rounding noise alone comes near the bar there (the
    whole-tensor bar still applies to it)."""
    # every element of every output is written (outputs were NaN-poisoned)
    for key, val in out.items():
        if val is not None:
            assert torch.isfinite(val).all().item(), f"{key}: non-finite (unwritten) elements"
    if full:
        ref = oracle.cref_backward(inp, d_out, d_final)
        H = inp["q"].shape[2]
        for key in TOKEN_GRADS + ("d_initial_state",):
            if out[key] is None:
                continue
            x = out[key].float().cpu().numpy().astype(np.float64)
            r = ref[key]
            ax = 2 if key in TOKEN_GRADS else 1
            worst = None
            for h in range(H):
                xh, rh = np.take(x, h, axis=ax), np.take(r, h, axis=ax)
                if rh.size < 4096:
                    break
                nr = np.linalg.norm(rh)
                if nr == 0.0:
                    assert not np.any(xh), (key, h)
                    continue
                rl2 = float(np.linalg.norm(xh - rh) / nr)
                mx = float(np.max(np.abs(xh - rh)) / np.max(np.abs(rh)))
                assert rl2 <= REL_L2 and mx <= MAX_REL, (key, h, rl2, mx)
                worst = rl2 if worst is None else max(worst, rl2)
            if worst is not None:
                print(f"{key}: worst head rel_l2={worst:.2e}", flush=True)
    else:
        ref = oracle.numpy_backward(inp, d_out, d_final)
    for key in TOKEN_GRADS:
        compare(key, out[key], ref[key])
    compare("dA_log", out["dA_log"], ref["dA_log"], alog_rel_l2)
    if out["ddt_bias"] is not None:
        compare("ddt_bias", out["ddt_bias"], ref["ddt_bias"])
    if out["d_initial_state"] is not None:
        compare("d_initial_state", out["d_initial_state"], ref["d_initial_state"])


@pytest.mark.parametrize("kw", [
    dict(B=1, T=64, H=2, initial_state=True),                     # whole chunks
    dict(B=2, T=37, H=3, initial_state=True),                     # ragged tail
    dict(B=1, T=16, H=1),                                         # one chunk, no state
    dict(B=3, T=1, H=2, initial_state=True),                      # one token per sequence
    dict(B=1, T=300, H=2, seq_lens=(0, 17, 1, 200, 82), initial_state=True),
    dict(B=1, T=333, H=4),                                        # many chunks, no state
])
def test_matches_oracle(kw):
    inp = kda_inputs.random_small(900 + kw["T"] + kw["H"], **kw)
    N = len(kw["seq_lens"]) if "seq_lens" in kw else kw["B"]
    d_out, d_final = kda_inputs.output_grads(901 + kw["T"], kw["B"], kw["T"], kw["H"], N=N)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final)


def test_without_final_gradient_or_optional_outputs():
    inp = kda_inputs.random_small(911, B=1, T=50, H=2, initial_state=True)
    d_out, _ = kda_inputs.output_grads(912, 1, 50, 2, final=False)
    out = run_bwd(to_device(inp), d_out, None, want_dtb=False, want_dinit=False)
    check(inp, out, d_out, None)


def test_fp32_initial_state_and_no_dt_bias():
    inp = kda_inputs.random_small(921, B=2, T=40, H=2, initial_state=True)
    inp["initial_state"] = inp["initial_state"].float() * 3.0
    inp["dt_bias"] = None
    d_out, d_final = kda_inputs.output_grads(922, 2, 40, 2)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final)


def test_strong_decay_at_the_lower_bound():
    # gates far beyond the bound: most tokens clamp, G reaches 16 x lower_bound
    inp = kda_inputs.random_small(931, B=1, T=48, H=2, initial_state=True, lower_bound=-5.4)
    inp["g"] = (inp["g"].float() + 4.0).to(torch.bfloat16)
    d_out, d_final = kda_inputs.output_grads(932, 1, 48, 2)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final)


def test_no_tokens():
    inp = kda_inputs.random_small(941, B=1, T=0, H=2, initial_state=True)
    d_out, d_final = kda_inputs.output_grads(942, 1, 0, 2)
    out = run_bwd(to_device(inp), d_out, d_final)
    assert torch.equal(out["dA_log"].cpu(), torch.zeros(2))
    assert torch.equal(out["ddt_bias"].cpu(), torch.zeros(2 * 128))
    assert torch.equal(out["d_initial_state"].cpu(), d_final)


def test_deterministic_bitwise():
    inp = kda_inputs.random_small(951, B=1, T=200, H=3, seq_lens=(70, 130), initial_state=True)
    d_out, d_final = kda_inputs.output_grads(952, 1, 200, 3, N=2)
    d = to_device(inp)
    a, b = run_bwd(d, d_out, d_final), run_bwd(d, d_out, d_final)
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.slow
def test_full_size_h96_all_heads():
    """T = 8192, H = 96 in the benchmark's launch configuration: every head's
    gradients against the C gradient oracle."""
    inp = kda_inputs.random_small(961, B=1, T=8192, H=96, initial_state=True)
    d_out, d_final = kda_inputs.output_grads(962, 1, 8192, 96)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final, full=True)


@pytest.mark.slow
def test_full_size_head_dim_256_all_heads():
    """T = 8192, H = 96 at K = V = 256 (the 256-wide kernels, as the
    benchmark runs them): every head's gradients against the C gradient
    oracle, dA_log to its 3e-2 bar at this width (see
    test_head_dim_256_matches_oracle)."""
    inp = kda_inputs.random_small(965, B=1, T=8192, H=96, K=256, V=256, initial_state=True)
    d_out, d_final = kda_inputs.output_grads(966, 1, 8192, 96, V=256, K=256)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final, alog_rel_l2=3e-2, full=True)


@pytest.mark.slow
def test_full_size_head_dim_64_all_heads():
    """T = 8192, H = 96 at K = V = 64 (the 64-wide kernels, as the benchmark
    runs them): every head's gradients against the C gradient oracle."""
    inp = kda_inputs.random_small(963, B=1, T=8192, H=96, K=64, V=64, initial_state=True)
    d_out, d_final = kda_inputs.output_grads(964, 1, 8192, 96, V=64, K=64)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final, full=True)


@pytest.mark.parametrize("kw", [
    dict(B=1, T=64, H=2, initial_state=True),
    dict(B=2, T=37, H=3),
    dict(B=1, T=300, H=2, seq_lens=(0, 17, 1, 200, 82), initial_state=True),
])
def test_head_dim_64_matches_oracle(kw):
    """K = V = 64 on the 64-wide kernels (5 KB states records, 7 KB reverse
    records, 64 x 64 stored states; the scans in two 32-column parts): every
    gradient against the oracle at K = V = 64."""
    inp = kda_inputs.random_small(950 + kw["T"] + kw["H"], K=64, V=64, **kw)
    N = len(kw["seq_lens"]) if "seq_lens" in kw else kw["B"]
    d_out, d_final = kda_inputs.output_grads(951 + kw["T"], kw["B"], kw["T"], kw["H"], V=64, N=N,
                                             K=64)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final)


def test_head_dim_64_one_part_scans():
    """K = V = 64 with N x H = 144 (sequence, head) units: the scans take one
    64-column part per unit (two scans of two parts would not fit on 256
    compute units); every head against the oracle."""
    inp = kda_inputs.random_small(931, B=2, T=150, H=72, K=64, V=64, initial_state=True)
    d_out, d_final = kda_inputs.output_grads(932, 2, 150, 72, V=64, K=64)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final, full=True)


@pytest.mark.parametrize("kw", [
    dict(B=1, T=64, H=2, initial_state=True),
    dict(B=2, T=37, H=3),
    dict(B=1, T=200, H=2, seq_lens=(0, 17, 1, 100, 82), initial_state=True),
])
def test_head_dim_256_matches_oracle(kw):
    """K = V = 256 on the 256-wide kernels (17 KB states records, 26 KB
    reverse records, 256 x 256 stored states; the scans in 32-column parts
    with one operand set per wave): every gradient against the oracle.

    dA_log is held to 3e-2 here instead of 5e-3: it is a sum over every
    (token, channel) whose terms cancel by a factor of up to about 230 on
    these inputs at K = 256 (about 30 at 128), and the bf16 records and
    stored states put 1.9e-2 of relative error on it in an fp64 restatement
    with the same roundings (tests/test_bwd_rounding_model.py; measured on
    the GPU: 2.0e-2); every other gradient keeps the 5e-3 bar."""
    inp = kda_inputs.random_small(910 + kw["T"] + kw["H"], K=256, V=256, **kw)
    N = len(kw["seq_lens"]) if "seq_lens" in kw else kw["B"]
    d_out, d_final = kda_inputs.output_grads(911 + kw["T"], kw["B"], kw["T"], kw["H"], V=256, N=N,
                                             K=256)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final, alog_rel_l2=3e-2)


def test_head_dim_256_edges():
    """K = V = 256: no d_final_state and no optional outputs; an fp32 initial
    state without dt_bias; no tokens (the initial-state gradient is d_final)."""
    inp = kda_inputs.random_small(941, B=1, T=50, H=2, K=256, V=256, initial_state=True)
    d_out, _ = kda_inputs.output_grads(942, 1, 50, 2, V=256, K=256, final=False)
    out = run_bwd(to_device(inp), d_out, None, want_dtb=False, want_dinit=False)
    check(inp, out, d_out, None, alog_rel_l2=3e-2)

    inp = kda_inputs.random_small(943, B=2, T=40, H=2, K=256, V=256, initial_state=True)
    inp["initial_state"] = inp["initial_state"].float() * 3.0
    inp["dt_bias"] = None
    d_out, d_final = kda_inputs.output_grads(944, 2, 40, 2, V=256, K=256)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final, alog_rel_l2=3e-2)

    inp = kda_inputs.random_small(945, B=1, T=0, H=2, K=256, V=256, initial_state=True)
    d_out, d_final = kda_inputs.output_grads(946, 1, 0, 2, V=256, K=256)
    out = run_bwd(to_device(inp), d_out, d_final)
    assert torch.equal(out["dA_log"].cpu(), torch.zeros(2))
    assert torch.equal(out["ddt_bias"].cpu(), torch.zeros(2 * 256))
    assert torch.equal(out["d_initial_state"].cpu(), d_final)


def test_head_dim_256_two_part_scans():
    """K = V = 256 with N x H = 48 units: the scans take 64-column parts (four
    per unit); every head against the oracle."""
    inp = kda_inputs.random_small(921, B=2, T=70, H=24, K=256, V=256, initial_state=True)
    d_out, d_final = kda_inputs.output_grads(922, 2, 70, 24, V=256, K=256)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final, alog_rel_l2=3e-2, full=True)


def test_many_heads():
    """N x H = 80 (sequence, head) units: ten groups of eight in the scans'
    XCD-aware block mapping; the two scans run side by side with one
    128-column part per unit (two scans of two parts would not fit on 256
    compute units at once)."""
    inp = kda_inputs.random_small(971, B=2, T=100, H=40, initial_state=True)
    d_out, d_final = kda_inputs.output_grads(972, 2, 100, 40)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final, full=True)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["varlen_mixed12_H96", "varlen_uniform_8x1024_H96"])
def test_full_size_varlen_all_heads(name):
    """The benchmark's varlen workloads at full size (8192 tokens, 96 heads):
    every head's gradients against the C gradient oracle."""
    w = kda_inputs.WORKLOADS[name]
    inp = kda_inputs.generate(w)
    d_out, d_final = kda_inputs.output_grads(w.seed + 1, w.B, w.T, w.H, N=w.num_seqs)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final, full=True)


def test_two_part_scans():
    """N x H = 48 (sequence, head) units: the scans take two 64-column parts
    per unit (2 scans x 2 parts x 48 fit on 256 compute units, four parts
    would not)."""
    inp = kda_inputs.random_small(991, B=2, T=50, H=24, initial_state=True)
    d_out, d_final = kda_inputs.output_grads(992, 2, 50, 24)
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final, full=True)


def test_many_units_with_empty_sequences():
    """200 (sequence, head) units, one 128-column part each; the batch
    holds empty and one-token sequences.  (Four-part scans, 32 columns per
    part, are what the small cases of test_matches_oracle take.)"""
    lens = (0, 17, 1, 60, 0)
    inp = kda_inputs.random_small(981, B=1, T=sum(lens), H=40, seq_lens=lens, initial_state=True)
    d_out, d_final = kda_inputs.output_grads(982, 1, sum(lens), 40, N=len(lens))
    out = run_bwd(to_device(inp), d_out, d_final)
    check(inp, out, d_out, d_final, full=True)
