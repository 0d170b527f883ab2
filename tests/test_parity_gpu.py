"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle on the
same seeded inputs, element by element.

Bar: o and final_state each within relative L2 <= 5e-3 and max-abs <= 3e-2
of the fp64 oracle; varlen index handling bit-exact (a sequence in a packed
batch gives bitwise the same o and final state as that sequence run alone).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
import oracle
from gpu_util import assert_close, np64, run_kda, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    kda.load()          # raises if the library is not built: no fallback
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def check_against_oracle(inp, out, fin, heads=None, use_c=True):
    if use_c:
        o_ref, f_ref = oracle.cref_forward(inp, heads=heads)
    else:
        o_ref, f_ref = oracle.numpy_forward(inp)
    o_gpu = np64(out)
    f_gpu = np64(fin) if fin is not None else None
    if heads is not None:
        o_gpu = o_gpu[:, :, heads]
        f_gpu = f_gpu[:, heads] if f_gpu is not None else None
    ro = assert_close("o", o_gpu, o_ref)
    rf = assert_close("final_state", f_gpu, f_ref) if f_gpu is not None else None
    print(f"o rel_l2={ro[0]:.3e} max_abs={ro[1]:.3e}"
          + (f"; final rel_l2={rf[0]:.3e} max_abs={rf[1]:.3e}" if rf else ""), flush=True)
    return ro, rf


def test_tiny_workload():
    inp = kda_inputs.generate(kda_inputs.WORKLOADS["tiny_T256_H2"])
    out, fin = run_kda(to_device(inp))
    check_against_oracle(inp, out, fin, use_c=False)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 100, 300])
def test_ragged_lengths_with_initial_state(T):
    inp = kda_inputs.random_small(100 + T, B=1, T=T, H=3, initial_state=True)
    out, fin = run_kda(to_device(inp))
    check_against_oracle(inp, out, fin)


def test_batched_fixed_length():
    inp = kda_inputs.random_small(7, B=3, T=37, H=5, initial_state=True)
    out, fin = run_kda(to_device(inp))
    check_against_oracle(inp, out, fin)


@pytest.mark.parametrize("B,H", [(1, 4), (1, 80), (2, 70)])
def test_scan_column_splits(B, H):
    """The scan splits each head's 128 columns over four, two or one
    workgroups depending on how many (sequence, head) units there are (at
    most 64, at most 128, more, on 256 compute units); one case of each."""
    inp = kda_inputs.random_small(900 + H, B=B, T=45, H=H, initial_state=True)
    out, fin = run_kda(to_device(inp))
    heads = sorted({0, H // 2, H - 1})
    check_against_oracle(inp, out, fin, heads=heads)


def test_varlen_with_empty_and_unit_sequences():
    inp = kda_inputs.random_small(8, B=1, T=100, H=4, seq_lens=[16, 1, 0, 33, 50, 0],
                                  initial_state=True)
    out, fin = run_kda(to_device(inp))
    check_against_oracle(inp, out, fin)
    # zero-length sequences hand their initial state through (bf16 -> fp32 exact)
    init = inp["initial_state"].float()
    assert torch.equal(fin[2].cpu(), init[2]) and torch.equal(fin[5].cpu(), init[5])


@pytest.mark.parametrize("init_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("final_dtype", [torch.bfloat16, torch.float32])
def test_state_dtypes(init_dtype, final_dtype):
    inp = kda_inputs.random_small(9, B=2, T=50, H=2, initial_state=True)
    inp["initial_state"] = inp["initial_state"].to(init_dtype)
    out, fin = run_kda(to_device(inp), final_dtype=final_dtype)
    check_against_oracle(inp, out, fin)


def test_null_initial_state_equals_zero_state_bitwise():
    inp = kda_inputs.random_small(10, B=1, T=70, H=3)
    d = to_device(inp)
    out0, fin0 = run_kda(d)
    zeros = torch.zeros(1, 3, 128, 128, dtype=torch.bfloat16, device="cuda")
    out1, fin1 = run_kda(d, initial_state=zeros)
    assert torch.equal(out0, out1) and torch.equal(fin0, fin1)


def test_final_state_optional():
    inp = kda_inputs.random_small(11, B=1, T=40, H=2, initial_state=True)
    d = to_device(inp)
    out0, _ = run_kda(d, want_final=False)
    out1, _ = run_kda(d)
    assert torch.equal(out0, out1)


def test_deterministic_bitwise():
    inp = kda_inputs.random_small(12, B=1, T=200, H=6, seq_lens=[70, 130], initial_state=True)
    d = to_device(inp)
    a = run_kda(d)
    b = run_kda(d)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_varlen_bitexact_against_single_sequences():
    lens = [5, 64, 0, 1, 47, 19]
    inp = kda_inputs.random_small(13, B=1, T=sum(lens), H=3, seq_lens=lens, initial_state=True)
    d = to_device(inp)
    out, fin = run_kda(d)
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        if e == s:
            continue
        sub = dict(d)
        for key in ("q", "k", "v", "g", "beta"):
            sub[key] = d[key][:, s:e].contiguous()
        sub["cu_seqlens"] = None
        sub["initial_state"] = d["initial_state"][n:n + 1].contiguous()
        o1, f1 = run_kda(sub)
        assert torch.equal(out[:, s:e], o1), f"sequence {n}: o differs"
        assert torch.equal(fin[n:n + 1], f1), f"sequence {n}: final state differs"


def test_uniform_varlen_bitexact_against_fixed_batch():
    B, T, H = 4, 48, 3
    inp = kda_inputs.random_small(14, B=1, T=B * T, H=H, seq_lens=[T] * B, initial_state=True)
    d = to_device(inp)
    out_v, fin_v = run_kda(d)
    fixed = dict(d)
    for key in ("q", "k", "v", "g", "beta"):
        fixed[key] = d[key].reshape((B, T) + tuple(d[key].shape[2:])).contiguous()
    fixed["cu_seqlens"] = None
    out_f, fin_f = run_kda(fixed)
    assert torch.equal(out_v.reshape(out_f.shape), out_f) and torch.equal(fin_v, fin_f)


# ------------------------------------------------------------------ edges
def test_all_gates_clamped_at_min_lower_bound():
    lb = kda.lower_bound_min()
    inp = kda_inputs.random_small(15, B=1, T=80, H=2, initial_state=True, lower_bound=lb)
    inp["g"] = torch.full_like(inp["g"], 80.0)
    out, fin = run_kda(to_device(inp))
    check_against_oracle(inp, out, fin)


def test_no_decay_alpha_one():
    inp = kda_inputs.random_small(16, B=1, T=90, H=2, initial_state=True)
    inp["A_log"] = torch.full_like(inp["A_log"], -math.inf)
    out, fin = run_kda(to_device(inp))
    check_against_oracle(inp, out, fin)


@pytest.mark.parametrize("T,A_log", [(65536, None), (32768, -math.inf)])
def test_long_sequence(T, A_log):
    """4096 chunk steps with the recipe's decay, and 2048 with none at all
    (alpha = 1: the fp32 state carries every update to the end): the state
    accumulated over the whole sequence stays within the parity bar."""
    inp = kda_inputs.random_small(23 + T, B=1, T=T, H=2, initial_state=True)
    if A_log is not None:
        inp["A_log"] = torch.full_like(inp["A_log"], A_log)
    out, fin = run_kda(to_device(inp))
    check_against_oracle(inp, out, fin)


@pytest.mark.parametrize("logit", [-math.inf, math.inf])
def test_beta_saturated(logit):
    inp = kda_inputs.random_small(17, B=1, T=60, H=2, initial_state=True)
    inp["beta"] = torch.full_like(inp["beta"], logit)
    # slow decay so that with beta = 0 the initial state is still visible at the end
    inp["A_log"] = torch.full_like(inp["A_log"], -3.0)
    out, fin = run_kda(to_device(inp))
    check_against_oracle(inp, out, fin)


def test_no_dt_bias():
    inp = kda_inputs.random_small(18, B=1, T=50, H=2, initial_state=True)
    inp["dt_bias"] = None
    out, fin = run_kda(to_device(inp))
    check_against_oracle(inp, out, fin)


def test_zero_tokens_passes_state_through():
    inp = kda_inputs.random_small(19, B=2, T=0, H=2, initial_state=True)
    out, fin = run_kda(to_device(inp))
    assert out.numel() == 0
    assert torch.equal(fin.cpu(), inp["initial_state"].float())


def test_invalid_arguments_raise():
    inp = kda_inputs.random_small(20, B=1, T=16, H=1)
    d = to_device(inp)
    out = torch.empty_like(d["v"])
    with pytest.raises(kda.KDAError):
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], out, d["A_log"],
                d["dt_bias"], -20.0)
    with pytest.raises(kda.KDAError):
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], float("nan"), out, d["A_log"],
                d["dt_bias"], -5.0)
