"""GPU parity of the decode step (kda_decode) against the fp64 oracle.

One decode step is the token recurrence for a single token from a given
state, so the oracle for it is the oracle forward over sequences of length
one with that state as the initial state.  A prefill of T tokens followed by
a decode step must match the oracle's prefill of T + 1 tokens.
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

# The step runs in fp32 from exact bf16 inputs: an fp32 state carries only
# fp32 rounding (about 1e-7 relative per operation over 128-term sums); the
# bf16 output and a bf16 state carry one bf16 rounding (2^-9 relative).
STATE_FP32_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    kda.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def single_token_inputs(seed, N, H, state_dtype, state_std=0.05, D=128):
    """N one-token sequences (B = N, T = 1) with a random initial state;
    head dimension K = V = D."""
    inp = kda_inputs.random_small(seed, B=N, T=1, H=H, K=D, V=D)
    gen = torch.Generator().manual_seed(10_000 + seed)
    st = torch.randn(N, H, D, D, generator=gen) * state_std
    inp["initial_state"] = st.to(state_dtype)
    return inp


def run_decode(inp, state):
    """kda.decode on device copies of a one-token-per-sequence input dict;
    `state` (device) is updated in place.  Returns out [N, H, V]."""
    d = to_device(inp)
    N, _, H, K = d["q"].shape
    flat = lambda t: t.reshape(N, H, -1).contiguous()
    out = torch.full((N, H, d["v"].shape[-1]), float("nan"), dtype=torch.bfloat16, device="cuda")
    kda.decode(flat(d["q"]), flat(d["k"]), flat(d["v"]), flat(d["g"]),
               d["beta"].reshape(N, H).contiguous(), d["scale"], out, d["A_log"],
               d.get("dt_bias"), d["lower_bound"], state)
    torch.cuda.synchronize()
    return out


def check(inp, out, state, state_tol=None, per_head=False):
    o_ref, f_ref = oracle.cref_forward(inp)
    o = np64(out)[:, None]                      # [N, 1, H, V] like the oracle's o
    f = np64(state)
    st = (lambda n, x, r: assert_close(n, x, r, rel_tol=state_tol)) if state_tol else assert_close
    ro = assert_close("o", o, o_ref)
    rf = st("state", f, f_ref)
    print(f"o rel_l2={ro[0]:.3e}; state rel_l2={rf[0]:.3e}", flush=True)
    if per_head:
        for h in range(o.shape[2]):
            assert_close(f"o head {h}", o[:, :, h], o_ref[:, :, h])
            st(f"state head {h}", f[:, h], f_ref[:, h])
    return ro, rf


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,H", [(1, 1), (3, 2), (17, 5)])
def test_decode_matches_oracle(N, H, state_dtype):
    inp = single_token_inputs(11 * N + H, N, H, state_dtype)
    state = inp["initial_state"].cuda()
    out = run_decode(inp, state)
    check(inp, out, state, state_tol=STATE_FP32_TOL if state_dtype == torch.float32 else None)


@pytest.mark.parametrize("T", [1, 16, 37])
def test_prefill_then_decode_equals_longer_prefill(T):
    full = kda_inputs.random_small(500 + T, B=1, T=T + 1, H=3, initial_state=True)
    head = {k: v for k, v in full.items()}
    for name in ("q", "k", "v", "g", "beta"):
        head[name] = full[name][:, :T].contiguous()
    # GPU prefill of the first T tokens, fp32 final state
    _, fin = run_kda(to_device(head), final_dtype=torch.float32)
    # GPU decode of token T from that state
    step = {k: v for k, v in full.items()}
    for name in ("q", "k", "v", "g", "beta"):
        step[name] = full[name][:, T:].contiguous()
    out = run_decode(step, fin)
    o_ref, f_ref = oracle.cref_forward(full)
    ro = assert_close("o", np64(out)[:, None], o_ref[:, T:])
    rf = assert_close("state", np64(fin), f_ref)
    print(f"T={T}: o rel_l2={ro[0]:.3e}; state rel_l2={rf[0]:.3e}", flush=True)


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_many_steps_equal_longer_prefill(state_dtype):
    """A 32-token prefill, then 256 decode steps one token at a time on the
    same state in place (fp32, or bf16 rounded after every step), against
    the oracle's prefill of all 288 tokens: every step's output and the final
    state."""
    P, S = 32, 256
    full = kda_inputs.random_small(777, B=2, T=P + S, H=3, initial_state=True)
    head = {k: v for k, v in full.items()}
    for name in ("q", "k", "v", "g", "beta"):
        head[name] = full[name][:, :P].contiguous()
    _, state = run_kda(to_device(head), final_dtype=state_dtype)
    outs = []
    for t in range(P, P + S):
        step = {k: v for k, v in full.items()}
        for name in ("q", "k", "v", "g", "beta"):
            step[name] = full[name][:, t:t + 1].contiguous()
        outs.append(run_decode(step, state))
    o_ref, f_ref = oracle.cref_forward(full)
    o = np.stack([np64(x) for x in outs], axis=1)           # [B, S, H, V]
    ro = assert_close("o", o, o_ref[:, P:])
    rf = assert_close("state", np64(state), f_ref)
    print(f"{state_dtype}: o rel_l2={ro[0]:.3e}; state rel_l2={rf[0]:.3e}", flush=True)


def test_no_decay_and_saturated_beta():
    inp = single_token_inputs(7, 4, 3, torch.float32)
    inp["A_log"] = torch.full_like(inp["A_log"], -math.inf)       # alpha = 1 exactly
    b = inp["beta"].clone()
    b[0] = math.inf                                                # beta = 1
    b[1] = -math.inf                                               # beta = 0: state only decays
    inp["beta"] = b
    state = inp["initial_state"].cuda()
    out = run_decode(inp, state)
    check(inp, out, state, state_tol=STATE_FP32_TOL)
    # beta = 0 and no decay leave the state of sequence 1 unchanged
    assert torch.equal(state[1].cpu(), inp["initial_state"][1])


@pytest.mark.parametrize("lb", [-5.0, -20.0, 0.0])
def test_gate_clamp_beyond_prefill_bound(lb):
    inp = single_token_inputs(31, 5, 2, torch.float32, state_std=1.0)
    inp["g"] = (inp["g"].float() * 0 + 40.0).to(torch.bfloat16)      # softplus ~ 40: clamped
    inp["lower_bound"] = lb
    state = inp["initial_state"].cuda()
    out = run_decode(inp, state)
    check(inp, out, state, state_tol=STATE_FP32_TOL)


def test_no_dt_bias():
    inp = single_token_inputs(41, 3, 4, torch.float32)
    inp["dt_bias"] = None
    state = inp["initial_state"].cuda()
    out = run_decode(inp, state)
    check(inp, out, state, state_tol=STATE_FP32_TOL)


def test_writes_only_its_state_and_output():
    inp = single_token_inputs(51, 3, 2, torch.float32)
    n = 3 * 2 * 128 * 128
    buf = torch.full((n + 2 * 4096,), 12345.0, device="cuda")
    state = buf[4096:4096 + n].view(3, 2, 128, 128)
    state.copy_(inp["initial_state"].cuda())
    out = run_decode(inp, state)
    assert torch.all(buf[:4096] == 12345.0) and torch.all(buf[4096 + n:] == 12345.0)
    check(inp, out, state, state_tol=STATE_FP32_TOL)


def test_deterministic_bitwise():
    inp = single_token_inputs(61, 6, 3, torch.float32)
    s1 = inp["initial_state"].cuda()
    s2 = inp["initial_state"].cuda()
    o1 = run_decode(inp, s1)
    o2 = run_decode(inp, s2)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_decode_batch64_h96_all_heads():
    """The measured configuration (64 sequences x 96 heads, fp32 state):
    every head against the oracle, each head also on its own."""
    inp = single_token_inputs(71, 64, 96, torch.float32)
    state = inp["initial_state"].cuda()
    out = run_decode(inp, state)
    check(inp, out, state, state_tol=STATE_FP32_TOL, per_head=True)


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("N,H", [(1, 1), (5, 3)])
def test_other_head_dims_match_oracle(D, N, H, state_dtype):
    """Head dimension 64 and 256: 64 and 1024 threads per (sequence, head)."""
    inp = single_token_inputs(31 * N + H + D, N, H, state_dtype, D=D)
    state = inp["initial_state"].cuda()
    out = run_decode(inp, state)
    check(inp, out, state, state_tol=STATE_FP32_TOL if state_dtype == torch.float32 else None)


@pytest.mark.parametrize("D", [64, 256])
def test_other_head_dims_prefill_then_decode(D):
    T = 37
    full = kda_inputs.random_small(600 + D, B=1, T=T + 1, H=2, K=D, V=D, initial_state=True)
    head = dict(full)
    step = dict(full)
    for name in ("q", "k", "v", "g", "beta"):
        head[name] = full[name][:, :T].contiguous()
        step[name] = full[name][:, T:].contiguous()
    _, fin = run_kda(to_device(head), final_dtype=torch.float32)
    out = run_decode(step, fin)
    o_ref, f_ref = oracle.cref_forward(full)
    ro = assert_close("o", np64(out)[:, None], o_ref[:, T:])
    rf = assert_close("state", np64(fin), f_ref)
    print(f"D={D}: o rel_l2={ro[0]:.3e}; state rel_l2={rf[0]:.3e}", flush=True)
