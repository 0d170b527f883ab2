"""GPU tests of the Gated DeltaNet form (kda_fwd_scalar_gate): one gate value
per (token, head) shared by all channels.

That form is the channel-wise forward on a gate broadcast over channels, so
(1) its results must equal kda_fwd's on broadcast g and dt_bias bit for bit,
and (2) the fp64 oracle on the broadcast inputs is its reference.
"""
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


def scalar_gate_inputs(seed, **kw):
    """Inputs with a per-(token, head) gate: g_s [B, T, H], dt_bias_s [H], and
    the same gate broadcast over channels in g [B, T, H, K], dt_bias [H*K]."""
    inp = kda_inputs.random_small(seed, **kw)
    g_s = inp["g"][..., 0].contiguous()
    gen = torch.Generator().manual_seed(20_000 + seed)
    H = g_s.shape[-1]
    dtb_s = torch.randn(H, generator=gen) * 0.5
    inp["g"] = g_s[..., None].expand(*g_s.shape, 128).contiguous()
    inp["dt_bias"] = dtb_s.repeat_interleave(128).contiguous()
    return inp, g_s, dtb_s


def run_scalar(inp, g_s, dtb_s, final_dtype=torch.float32):
    d = to_device(inp)
    B, T, H, _ = d["q"].shape
    cu = d.get("cu_seqlens")
    N = B if cu is None else cu.numel() - 1
    out = torch.full((B, T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((N, H, 128, 128), float("nan"), dtype=final_dtype, device="cuda")
    kda.fwd_scalar_gate(d["q"], d["k"], d["v"], g_s.cuda(), d["beta"], d["scale"], out,
                        d["A_log"], None if dtb_s is None else dtb_s.cuda(), d["lower_bound"],
                        initial_state=d.get("initial_state"), final_state=fin, cu_seqlens=cu)
    torch.cuda.synchronize()
    return out, fin


CASES = [
    dict(B=1, T=256, H=2),
    dict(B=1, T=37, H=3, initial_state=True),
    dict(B=2, T=100, H=2, initial_state=True),
    dict(B=1, T=300, H=3, seq_lens=(0, 17, 1, 200, 82), initial_state=True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_bitwise_equal_to_channelwise_on_broadcast_gate(case):
    inp, g_s, dtb_s = scalar_gate_inputs(300 + case, **CASES[case])
    out_s, fin_s = run_scalar(inp, g_s, dtb_s)
    out_c, fin_c = run_kda(to_device(inp))
    assert torch.equal(out_s, out_c)
    assert torch.equal(fin_s, fin_c)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_matches_oracle(case):
    inp, g_s, dtb_s = scalar_gate_inputs(400 + case, **CASES[case])
    out, fin = run_scalar(inp, g_s, dtb_s)
    o_ref, f_ref = oracle.cref_forward(inp)
    ro = assert_close("o", np64(out), o_ref)
    rf = assert_close("final_state", np64(fin), f_ref)
    print(f"o rel_l2={ro[0]:.3e}; final rel_l2={rf[0]:.3e}", flush=True)


def test_no_dt_bias_and_clamped_gates():
    inp, g_s, _ = scalar_gate_inputs(501, B=1, T=64, H=2, initial_state=True)
    g_s = (g_s.float() * 0 + 30.0).to(torch.bfloat16)      # softplus ~ 30: every gate clamped
    inp["g"] = g_s[..., None].expand(*g_s.shape, 128).contiguous()
    inp["dt_bias"] = None
    inp["lower_bound"] = kda.lower_bound_min()
    out, fin = run_scalar(inp, g_s, None)
    o_ref, f_ref = oracle.cref_forward(inp)
    assert_close("o", np64(out), o_ref)
    assert_close("final_state", np64(fin), f_ref)


@pytest.mark.slow
def test_full_size_h96_all_heads():
    """T = 8192, H = 96 with the scalar gate, every head against the oracle."""
    inp, g_s, dtb_s = scalar_gate_inputs(601, B=1, T=8192, H=96, initial_state=True)
    out, fin = run_scalar(inp, g_s, dtb_s)
    o_ref, f_ref = oracle.cref_forward(inp)
    ro = assert_close("o", np64(out), o_ref)
    rf = assert_close("final_state", np64(fin), f_ref)
    print(f"o rel_l2={ro[0]:.3e}; final rel_l2={rf[0]:.3e}", flush=True)
