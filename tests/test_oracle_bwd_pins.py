"""Pins for the fp64 gradient oracle (oracle/kda_ref_bwd.py), never against
itself:

  * central finite differences of the forward oracle's loss
    L = <d_out, o> + <d_final, final_state> for every element of every input
    (q, k, v, g, beta logits, A_log, dt_bias, initial state), on a fixed-length
    batch and on a varlen batch with an empty sequence, with tokens on both
    sides of the gate clamp;
  * two exact identities of the forward: o and the final state are linear in
    (v, initial state) jointly, so <v, dv> + <S0, dS0> = L; and o is linear
    in q while the states do not depend on q, so <q, dq> = <d_out, o>.

A dropped term of the adjoint step (the k dw^T or S' dw pieces, the decay on
dS, the gate chain, the sigmoid derivative) or a wrong sign moves a gradient
far outside the finite-difference bound; a state that is not reset per
sequence fails the varlen case.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import kda_inputs
import oracle

H, K, V = 2, 3, 2
LB = -2.0


def make_case(seed, B, T, N, cu=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    A_log = np.log(rng.uniform(1, 4, size=H))
    dt_bias = 0.1 * rng.standard_normal(H * K)
    g = rng.standard_normal((B, T, H, K))
    # keep every gate value at least 0.05 away from the clamp, on either side,
    # so that a finite difference never straddles it
    A = np.exp(A_log).reshape(H, 1)
    for _ in range(100):
        y = -A * np.logaddexp(0.0, g + dt_bias.reshape(H, K))
        near = np.abs(y - LB) < 0.05
        if not near.any():
            break
        g = np.where(near, g - 0.2, g)
    c = dict(q=q, k=k, v=rng.standard_normal((B, T, H, V)), g=g,
             beta=rng.standard_normal((B, T, H)), A_log=A_log, dt_bias=dt_bias,
             initial_state=0.5 * rng.standard_normal((N, H, K, V)))
    d_out = rng.standard_normal((B, T, H, V))
    d_final = rng.standard_normal((N, H, K, V))
    return c, d_out, d_final, cu


def loss(c, d_out, d_final, cu):
    o, fin = oracle.kda_forward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["A_log"],
                                c["dt_bias"], LB, 1.0 / math.sqrt(K),
                                initial_state=c["initial_state"], cu_seqlens=cu)
    return float(np.sum(d_out * o) + np.sum(d_final * fin)), o, fin


def grads(c, d_out, d_final, cu, checkpoint=64):
    return oracle.kda_backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["A_log"],
                               c["dt_bias"], LB, 1.0 / math.sqrt(K), d_out, d_final=d_final,
                               initial_state=c["initial_state"], cu_seqlens=cu,
                               checkpoint=checkpoint)


NAMES = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
         ("A_log", "dA_log"), ("dt_bias", "ddt_bias"), ("initial_state", "d_initial_state")]


@pytest.mark.parametrize("case", ["fixed_B2", "varlen_with_empty"])
def test_finite_differences_every_input(case):
    if case == "fixed_B2":
        c, d_out, d_final, cu = make_case(11, B=2, T=5, N=2)
    else:
        c, d_out, d_final, cu = make_case(12, B=1, T=7, N=3, cu=np.array([0, 2, 2, 7]))
    gr = grads(c, d_out, d_final, cu, checkpoint=3)
    # both sides of the clamp are present
    y = -np.exp(c["A_log"]).reshape(H, 1) * np.logaddexp(0.0, c["g"] + c["dt_bias"].reshape(H, K))
    assert (y < LB).any() and (y > LB).any()
    assert np.all(gr["dg"][y < LB] == 0.0)
    h = 1e-6
    for name, gname in NAMES:
        x = c[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = loss(c, d_out, d_final, cu)[0]
            x[idx] = old - h
            lm = loss(c, d_out, d_final, cu)[0]
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        got = gr[gname].reshape(fd.shape)
        err = np.max(np.abs(got - fd))
        assert err <= 1e-7 + 1e-6 * np.max(np.abs(fd)), (name, err)
        assert np.max(np.abs(fd)) > 1e-3, name        # the check is not vacuous


def test_linearity_identities():
    rng_case = make_case(21, B=1, T=40, N=3, cu=np.array([0, 13, 13, 40]))
    c, d_out, d_final, cu = rng_case
    L, o, _ = loss(c, d_out, d_final, cu)
    gr = grads(c, d_out, d_final, cu, checkpoint=5)
    lhs = np.sum(c["v"] * gr["dv"]) + np.sum(c["initial_state"] * gr["d_initial_state"])
    assert abs(lhs - L) <= 1e-11 * max(1.0, abs(L))
    assert abs(np.sum(c["q"] * gr["dq"]) - np.sum(d_out * o)) <= 1e-11 * max(1.0, abs(L))


def test_checkpoint_spacing_changes_nothing():
    c, d_out, d_final, cu = make_case(31, B=2, T=11, N=2)
    a = grads(c, d_out, d_final, cu, checkpoint=1)
    for cp in (3, 64):
        b = grads(c, d_out, d_final, cu, checkpoint=cp)
        for key in a:
            np.testing.assert_allclose(b[key], a[key], rtol=1e-13, atol=1e-15)


def test_no_final_gradient_and_no_initial_state():
    c, d_out, d_final, cu = make_case(41, B=1, T=6, N=1)
    c["initial_state"] = None
    gr = oracle.kda_backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["A_log"],
                             c["dt_bias"], LB, 1.0 / math.sqrt(K), d_out)
    # with a zero initial state, d_out alone: the last token's q gradient is
    # scale * S_T d_out_T (the output is read from the updated state)
    o, fin = oracle.kda_forward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["A_log"],
                                c["dt_bias"], LB, 1.0 / math.sqrt(K))
    want = np.einsum("hkv,hv->hk", fin[0], d_out[0, -1]) / math.sqrt(K)
    np.testing.assert_allclose(gr["dq"][0, -1], want, rtol=1e-12, atol=1e-14)


def test_head_subset_matches_full():
    inp = kda_inputs.random_small(5, B=1, T=20, H=3, K=8, V=8, seq_lens=(7, 13),
                                  initial_state=True)
    d_out, d_final = kda_inputs.output_grads(6, 1, 20, 3, V=8, N=2, K=8)
    full = oracle.numpy_backward(inp, d_out, d_final)
    sub = oracle.numpy_backward(inp, d_out, d_final, heads=[2, 0])
    for key in ("dq", "dk", "dv", "dg"):
        np.testing.assert_array_equal(sub[key], full[key][:, :, [2, 0]])
    np.testing.assert_array_equal(sub["dbeta"], full["dbeta"][:, :, [2, 0]])
    np.testing.assert_array_equal(sub["dA_log"], full["dA_log"][[2, 0]])
    np.testing.assert_array_equal(sub["ddt_bias"].reshape(2, 8),
                                  full["ddt_bias"].reshape(3, 8)[[2, 0]])
    np.testing.assert_array_equal(sub["d_initial_state"], full["d_initial_state"][:, [2, 0]])


@pytest.mark.parametrize("case", [
    dict(kw=dict(B=1, T=300, H=2, seq_lens=(0, 17, 1, 200, 82), initial_state=True)),
    dict(kw=dict(B=2, T=70, H=3, initial_state=True), fp32_init=True, no_dtb=True, no_final=True),
    dict(kw=dict(B=1, T=48, H=2, initial_state=True, lower_bound=-5.4), gate_shift=4.0),
    dict(kw=dict(B=1, T=90, H=4, initial_state=True), heads=[3, 1]),
    dict(kw=dict(B=1, T=40, H=2, K=64, V=64, initial_state=True)),
    dict(kw=dict(B=1, T=20, H=1, K=256, V=256, initial_state=True)),
    dict(kw=dict(B=1, T=0, H=2, initial_state=True)),
])
def test_c_gradient_oracle_matches_numpy(case):
    """The C restatement of the gradient oracle (cref_backward, for full
    sizes) gives the numpy oracle's gradients, which the tests above pin by
    finite differences, to rounding order: ragged varlen with empty and
    one-token sequences, fp32 initial state without dt_bias or d_final, gates
    clamped at the lowest lower bound, a head subset in a given order, head
    dimensions 64 and 256, and no tokens."""
    kw = case["kw"]
    inp = kda_inputs.random_small(1300 + kw["T"] + kw["H"], **kw)
    if case.get("fp32_init"):
        inp["initial_state"] = inp["initial_state"].float() * 2.0
    if case.get("no_dtb"):
        inp["dt_bias"] = None
    if case.get("gate_shift"):
        inp["g"] = (inp["g"].float() + case["gate_shift"]).to(torch.bfloat16)
    N = len(kw["seq_lens"]) if "seq_lens" in kw else kw["B"]
    K = kw.get("K", 128)
    d_out, d_final = kda_inputs.output_grads(1301 + kw["T"], kw["B"], kw["T"], kw["H"], V=K, N=N,
                                             K=K)
    if case.get("no_final"):
        d_final = None
    heads = case.get("heads")
    ref = oracle.numpy_backward(inp, d_out, d_final, heads=heads)
    got = oracle.cref_backward(inp, d_out, d_final, heads=heads, threads=4)
    for key, r in ref.items():
        r = np.asarray(r)
        x = got[key]
        assert x.shape == r.shape, key
        nr = np.linalg.norm(r)
        if nr == 0.0:
            assert not np.any(x), key
            continue
        assert np.linalg.norm(x - r) / nr < 1e-11, (key, np.linalg.norm(x - r) / nr)
