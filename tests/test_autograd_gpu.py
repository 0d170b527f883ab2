"""kda.attention, the differentiable wrapper: its forward is kda_fwd and its
gradients are kda_bwd's, bit for bit, on the incoming gradients autograd
hands it (the parity of both entries against the oracle is covered by the
forward and backward parity tests)."""
from __future__ import annotations

import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
from gpu_util import to_device

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "beta", "A_log", "dt_bias")


def leaves(d, init=None):
    x = {n: d[n].clone().requires_grad_(True) for n in NAMES if d.get(n) is not None}
    if init is not None:
        x["initial_state"] = init.clone().requires_grad_(True)
    return x


def direct(d, d_out, d_final, init):
    """kda.fwd and kda.bwd called directly on the same inputs."""
    B, T, H, K = d["q"].shape
    V = d["v"].shape[-1]
    cu = d.get("cu_seqlens")
    N = B if cu is None else cu.numel() - 1
    o = torch.empty((B, T, H, V), dtype=torch.bfloat16, device="cuda")
    fs = torch.empty((N, H, K, V), dtype=torch.float32, device="cuda")
    kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], o, d["A_log"], d.get("dt_bias"),
            d["lower_bound"], initial_state=init, final_state=fs, cu_seqlens=cu)
    gr = {n: torch.empty_like(d[n]) for n in NAMES if d.get(n) is not None}
    di = None if init is None else torch.empty(init.shape, dtype=torch.float32, device="cuda")
    kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"], d.get("dt_bias"),
            d["lower_bound"], d_out, gr["q"], gr["k"], gr["v"], gr["g"], gr["beta"], gr["A_log"],
            ddt_bias=gr.get("dt_bias"), initial_state=init, d_final_state=d_final,
            d_initial_state=di, cu_seqlens=cu)
    if di is not None:
        gr["initial_state"] = di.to(init.dtype)
    return o, fs, gr


@pytest.mark.parametrize("init_dtype", [None, torch.float32, torch.bfloat16])
def test_gradients_equal_direct_calls(init_dtype):
    inp = kda_inputs.random_small(620, B=1, T=150, H=3, seq_lens=(0, 40, 1, 109),
                                  initial_state=init_dtype is not None)
    d = to_device(inp)
    init = None if init_dtype is None else d["initial_state"].to(init_dtype)
    d_out, d_final = kda_inputs.output_grads(621, 1, 150, 3, N=4)
    d_out, d_final = d_out.cuda(), d_final.cuda()
    x = leaves(d, init)
    o, fs = kda.attention(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["dt_bias"],
                          d["lower_bound"], scale=d["scale"], initial_state=x.get("initial_state"),
                          output_final_state=True, cu_seqlens=d["cu_seqlens"])
    loss = (o.float() * d_out.float()).sum() + (fs * d_final).sum()
    loss.backward()
    o_ref, fs_ref, gr = direct(d, d_out, d_final, init)
    assert torch.equal(o, o_ref) and torch.equal(fs, fs_ref)
    for n, t in x.items():
        assert t.grad is not None and t.grad.dtype == t.dtype, n
        assert torch.equal(t.grad, gr[n]), n


def test_output_only_and_default_scale():
    """No final state requested (its gradient is absent), no initial state,
    a fixed-length batch of two, scale left to its default K^-1/2."""
    inp = kda_inputs.random_small(622, B=2, T=48, H=2)
    d = to_device(inp)
    d_out, _ = kda_inputs.output_grads(623, 2, 48, 2, final=False)
    d_out = d_out.cuda()
    x = leaves(d)
    o, fs = kda.attention(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["dt_bias"],
                          d["lower_bound"])
    assert fs is None
    (o.float() * d_out.float()).sum().backward()
    d["scale"] = 128 ** -0.5
    o_ref, _, gr = direct(d, d_out, None, None)
    assert torch.equal(o, o_ref)
    for n, t in x.items():
        assert torch.equal(t.grad, gr[n]), n


def test_scalar_gate_form():
    """A gate of shape [B, T, H] selects the Gated DeltaNet form: outputs and
    gradients equal to fwd_scalar_gate and bwd_scalar_gate called directly."""
    inp = kda_inputs.random_small(624, B=1, T=70, H=2, seq_lens=(30, 40), initial_state=True)
    d = to_device(inp)
    d["g"] = d["g"][..., 0].contiguous()
    d["dt_bias"] = d["dt_bias"].view(2, -1)[:, 0].contiguous()
    init = d["initial_state"].float()
    d_out, d_final = kda_inputs.output_grads(625, 1, 70, 2, N=2)
    d_out, d_final = d_out.cuda(), d_final.cuda()
    x = leaves(d, init)
    o, fs = kda.attention(x["q"], x["k"], x["v"], x["g"], x["beta"], x["A_log"], x["dt_bias"],
                          d["lower_bound"], scale=d["scale"], initial_state=x["initial_state"],
                          output_final_state=True, cu_seqlens=d["cu_seqlens"])
    ((o.float() * d_out.float()).sum() + (fs * d_final).sum()).backward()
    o_ref = torch.empty_like(o)
    fs_ref = torch.empty_like(fs)
    kda.fwd_scalar_gate(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], o_ref, d["A_log"],
                        d["dt_bias"], d["lower_bound"], initial_state=init, final_state=fs_ref,
                        cu_seqlens=d["cu_seqlens"])
    gr = {n: torch.empty_like(d[n]) for n in NAMES}
    gr["initial_state"] = torch.empty_like(init)
    kda.bwd_scalar_gate(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"],
                        d["dt_bias"], d["lower_bound"], d_out, gr["q"], gr["k"], gr["v"], gr["g"],
                        gr["beta"], gr["A_log"], ddt_bias=gr["dt_bias"], initial_state=init,
                        d_final_state=d_final, d_initial_state=gr["initial_state"],
                        cu_seqlens=d["cu_seqlens"])
    assert torch.equal(o, o_ref) and torch.equal(fs, fs_ref)
    for n, t in x.items():
        assert torch.equal(t.grad, gr[n]), n
