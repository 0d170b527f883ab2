"""Full-size parity on the T=8192, D=128 workloads, in the same launch
configuration the benchmark times (kda.fwd with its defaults).

The C oracle computes every head (all 8192 tokens of each, about a second
on the host's cores) and the whole GPU output is compared element by
element.  The uniform varlen workload is also checked bitwise
against the same tokens run as a fixed-length batch of 8 x 1024.
"""
from __future__ import annotations

import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
import oracle
from gpu_util import assert_close, np64, run_kda, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("name", ["fixed_T8192_H64", "fixed_T8192_H96",
                                  "varlen_uniform_8x1024_H96", "varlen_mixed12_H96",
                                  "varlen_mixed12_H64"])
def test_full_size_workload(name):
    kda.load()
    w = kda_inputs.WORKLOADS[name]
    inp = kda_inputs.generate(w)
    d = to_device(inp)
    out, fin = run_kda(d)
    o_ref, f_ref = oracle.cref_forward(inp)
    o_gpu = np64(out)
    f_gpu = np64(fin)
    r_o = assert_close(f"{name} o", o_gpu, o_ref)
    r_f = assert_close(f"{name} final_state", f_gpu, f_ref)
    print(f"{name}: o rel_l2={r_o[0]:.3e} max_abs={r_o[1]:.3e}; "
          f"final rel_l2={r_f[0]:.3e} max_abs={r_f[1]:.3e}", flush=True)
    # per-head bar too, so that one wrong head cannot hide in the whole-tensor norm
    for h in range(w.H):
        assert_close(f"{name} o head {h}", o_gpu[:, :, h], o_ref[:, :, h])
        assert_close(f"{name} final_state head {h}", f_gpu[:, h], f_ref[:, h])
    if name == "varlen_uniform_8x1024_H96":
        fixed = dict(d)
        for key in ("q", "k", "v", "g", "beta"):
            fixed[key] = d[key].reshape((8, 1024) + tuple(d[key].shape[2:])).contiguous()
        fixed["cu_seqlens"] = None
        out_f, fin_f = run_kda(fixed)
        assert torch.equal(out.reshape(out_f.shape), out_f)
        assert torch.equal(fin, fin_f)


def test_long_sequence_split_bitexact():
    """T = 2^18 tokens on 2 heads.  The first 4096 output rows against the
    oracle (they depend only on the first 4096 tokens), and the run split at
    a chunk boundary: the second half started from the first half's fp32
    final state must reproduce the full run's second half and final state
    bit for bit (the scan keeps exactly that fp32 state at the boundary)."""
    T, H, P = 1 << 18, 2, 4096
    inp = kda_inputs.random_small(1001, B=1, T=T, H=H, initial_state=True)
    d = to_device(inp)
    out, fin = run_kda(d)
    assert torch.isfinite(out).all().item() and torch.isfinite(fin).all().item()
    pre = {key: (val[:, :P].contiguous() if key in ("q", "k", "v", "g", "beta") else val)
           for key, val in inp.items()}
    o_ref, _ = oracle.cref_forward(pre, want_final=False)
    assert_close("o[:4096]", np64(out[:, :P]), o_ref)
    half = T // 2
    first = {key: (val[:, :half].contiguous() if key in ("q", "k", "v", "g", "beta") else val)
             for key, val in d.items()}
    _, fin1 = run_kda(first, final_dtype=torch.float32)
    second = {key: (val[:, half:].contiguous() if key in ("q", "k", "v", "g", "beta") else val)
              for key, val in d.items()}
    second["initial_state"] = fin1
    out2, fin2 = run_kda(second, final_dtype=torch.float32)
    assert torch.equal(out[:, half:], out2)
    assert torch.equal(fin, fin2)


def test_many_heads():
    """H = 4096 heads (one column part per head in the scan), every head
    against the oracle."""
    H = 4096
    inp = kda_inputs.random_small(1002, B=1, T=40, H=H, initial_state=True)
    out, fin = run_kda(to_device(inp))
    o_ref, f_ref = oracle.cref_forward(inp)
    assert_close("o", np64(out), o_ref)
    assert_close("final_state", np64(fin), f_ref)
