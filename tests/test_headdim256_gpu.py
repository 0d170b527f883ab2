"""GPU parity of the forward at head dimension K = V = 256 against the fp64
oracle (which takes any K, V).  The kernels run on 256-wide tiles: sixteen
state row tiles per 16-column slice and 26 KB hand-off records."""
from __future__ import annotations

import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
import oracle
from gpu_util import assert_close, np64, run_kda, to_device

pytestmark = pytest.mark.gpu

D = 256


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    kda.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def check(inp, out, fin, per_head=False):
    """Every head against the C oracle; per_head: each head also on its own
    (the full-size case), so that one wrong head cannot hide in the norm."""
    o_ref, f_ref = oracle.cref_forward(inp)
    o, f = np64(out), np64(fin)
    ro = assert_close("o", o, o_ref)
    rf = assert_close("final_state", f, f_ref)
    print(f"o rel_l2={ro[0]:.3e}; final rel_l2={rf[0]:.3e}", flush=True)
    if per_head:
        for h in range(o.shape[2]):
            assert_close(f"o head {h}", o[:, :, h], o_ref[:, :, h])
            assert_close(f"final_state head {h}", f[:, h], f_ref[:, h])


@pytest.mark.parametrize("kw", [
    dict(B=1, T=256, H=2),                                   # eight 32-column parts per head
    dict(B=1, T=37, H=3, initial_state=True),                # ragged tail
    dict(B=2, T=100, H=2, initial_state=True),
    dict(B=1, T=300, H=3, seq_lens=(0, 17, 1, 200, 82), initial_state=True),
    dict(B=1, T=45, H=40, initial_state=True),               # four 64-column parts per head
    dict(B=2, T=60, H=40, initial_state=True),               # 80 units: two 128-column parts per head
    dict(B=1, T=16, H=1),                                    # one full chunk
])
def test_matches_oracle(kw):
    inp = kda_inputs.random_small(900 + kw["H"] + kw["T"], K=D, V=D, **kw)
    out, fin = run_kda(to_device(inp))
    check(inp, out, fin)


@pytest.mark.parametrize("final_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("init_dtype", [torch.bfloat16, torch.float32])
def test_state_dtypes(final_dtype, init_dtype):
    inp = kda_inputs.random_small(951, B=2, T=50, H=2, K=D, V=D, initial_state=True)
    d = to_device(inp)
    init = d["initial_state"].to(init_dtype)
    out, fin = run_kda(d, final_dtype=final_dtype, initial_state=init)
    check(inp, out, fin)


def test_no_initial_state_equals_zeros_bitwise():
    inp = kda_inputs.random_small(961, B=1, T=70, H=2, K=D, V=D)
    d = to_device(inp)
    a = run_kda(d, initial_state=None)
    z = torch.zeros(1, 2, D, D, dtype=torch.bfloat16, device="cuda")
    b = run_kda(d, initial_state=z)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_varlen_equals_single_sequence_runs_bitwise():
    lens = (40, 0, 77, 16, 3)
    inp = kda_inputs.random_small(971, B=1, T=sum(lens), H=3, K=D, V=D, seq_lens=lens,
                                  initial_state=True)
    d = to_device(inp)
    out, fin = run_kda(d)
    start = 0
    for n, L in enumerate(lens):
        if L:
            one = {key: (val[:, start:start + L].contiguous()
                         if key in ("q", "k", "v", "g", "beta") else val) for key, val in d.items()}
            one["cu_seqlens"] = None
            one["initial_state"] = d["initial_state"][n:n + 1].contiguous()
            o1, f1 = run_kda(one)
            assert torch.equal(out[:, start:start + L], o1), n
            assert torch.equal(fin[n:n + 1], f1), n
        else:
            assert torch.equal(fin[n].float(), d["initial_state"][n].float()), n
        start += L


def test_split_at_chunk_boundary_bitwise():
    """Two calls chained through an fp32 final state equal one call, bit for
    bit, when the split falls on a chunk boundary."""
    inp = kda_inputs.random_small(981, B=1, T=96, H=2, K=D, V=D, initial_state=True)
    d = to_device(inp)
    out, fin = run_kda(d)
    t1 = 48
    first = {key: (val[:, :t1].contiguous() if key in ("q", "k", "v", "g", "beta") else val)
             for key, val in d.items()}
    o1, f1 = run_kda(first)
    second = {key: (val[:, t1:].contiguous() if key in ("q", "k", "v", "g", "beta") else val)
              for key, val in d.items()}
    o2, f2 = run_kda(second, initial_state=f1)
    assert torch.equal(out[:, :t1], o1) and torch.equal(out[:, t1:], o2)
    assert torch.equal(fin, f2)


def test_scalar_gate_bitwise_with_broadcast_gate():
    inp = kda_inputs.random_small(991, B=1, T=120, H=3, K=D, V=D, initial_state=True)
    g_s = inp["g"][..., 0].contiguous()
    inp["g"] = g_s[..., None].expand(*g_s.shape, D).contiguous()
    dtb_s = torch.linspace(-0.5, 0.5, 3)
    inp["dt_bias"] = dtb_s.repeat_interleave(D).contiguous()
    d = to_device(inp)
    out = torch.full((1, 120, 3, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((1, 3, D, D), float("nan"), device="cuda")
    kda.fwd_scalar_gate(d["q"], d["k"], d["v"], g_s.cuda(), d["beta"], d["scale"], out, d["A_log"],
                        dtb_s.cuda(), d["lower_bound"], initial_state=d["initial_state"], final_state=fin)
    torch.cuda.synchronize()
    check(inp, out, fin)
    out_c, fin_c = run_kda(d)
    assert torch.equal(out, out_c) and torch.equal(fin, fin_c)


def test_all_gates_at_lower_bound():
    """Every gate clamped at the smallest supported lower bound (the largest
    in-chunk decay range the factorised gating must hold)."""
    lb = kda.lower_bound_min()
    inp = kda_inputs.random_small(1001, B=1, T=64, H=2, K=D, V=D, initial_state=True,
                                  lower_bound=lb)
    inp["g"] = torch.full_like(inp["g"], 30.0)
    inp["A_log"] = torch.full_like(inp["A_log"], 3.0)
    out, fin = run_kda(to_device(inp))
    check(inp, out, fin)


def test_deterministic_bitwise():
    inp = kda_inputs.random_small(1011, B=1, T=200, H=4, K=D, V=D, seq_lens=(70, 130),
                                  initial_state=True)
    d = to_device(inp)
    a, b = run_kda(d), run_kda(d)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.slow
def test_full_size_h96_all_heads():
    inp = kda_inputs.random_small(1021, B=1, T=8192, H=96, K=D, V=D, initial_state=True)
    out, fin = run_kda(to_device(inp))
    check(inp, out, fin, per_head=True)
