"""GPU parity of the forward at head dimension K = V = 64 against the fp64
oracle (which takes any K, V).  The kernels run on their 128-wide tiles with
the key channels and value columns from 64 on held at zero."""
from __future__ import annotations

import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
import oracle
from gpu_util import assert_close, np64, run_kda, to_device

pytestmark = pytest.mark.gpu


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
    dict(B=1, T=256, H=2),                                   # two 32-column parts per head
    dict(B=1, T=37, H=3, initial_state=True),
    dict(B=2, T=100, H=2, initial_state=True),
    dict(B=1, T=300, H=3, seq_lens=(0, 17, 1, 200, 82), initial_state=True),
    dict(B=1, T=45, H=200, initial_state=True),              # one 64-column part per head
])
def test_matches_oracle(kw):
    inp = kda_inputs.random_small(700 + kw["H"] + kw["T"], K=64, V=64, **kw)
    out, fin = run_kda(to_device(inp))
    check(inp, out, fin)


@pytest.mark.parametrize("final_dtype", [torch.bfloat16, torch.float32])
def test_state_dtypes_and_bf16_initial_state(final_dtype):
    inp = kda_inputs.random_small(801, B=2, T=50, H=2, K=64, V=64, initial_state=True)
    out, fin = run_kda(to_device(inp), final_dtype=final_dtype)
    check(inp, out, fin)


def test_scalar_gate():
    inp = kda_inputs.random_small(811, B=1, T=120, H=3, K=64, V=64, initial_state=True)
    g_s = inp["g"][..., 0].contiguous()
    inp["g"] = g_s[..., None].expand(*g_s.shape, 64).contiguous()
    dtb_s = torch.linspace(-0.5, 0.5, 3)
    inp["dt_bias"] = dtb_s.repeat_interleave(64).contiguous()
    d = to_device(inp)
    out = torch.full((1, 120, 3, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((1, 3, 64, 64), float("nan"), device="cuda")
    kda.fwd_scalar_gate(d["q"], d["k"], d["v"], g_s.cuda(), d["beta"], d["scale"], out, d["A_log"],
                        dtb_s.cuda(), d["lower_bound"], initial_state=d["initial_state"], final_state=fin)
    torch.cuda.synchronize()
    check(inp, out, fin)
    out_c, fin_c = run_kda(d)
    assert torch.equal(out, out_c) and torch.equal(fin, fin_c)


def test_deterministic_bitwise():
    inp = kda_inputs.random_small(821, B=1, T=200, H=4, K=64, V=64, seq_lens=(70, 130),
                                  initial_state=True)
    d = to_device(inp)
    a, b = run_kda(d), run_kda(d)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.slow
def test_full_size_h96_all_heads():
    inp = kda_inputs.random_small(831, B=1, T=8192, H=96, K=64, V=64, initial_state=True)
    out, fin = run_kda(to_device(inp))
    check(inp, out, fin, per_head=True)
