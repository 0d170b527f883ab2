"""Pins for the fp64 oracle: it is checked against hand-worked values, closed
forms, special cases that reduce to textbook operations, invariants and
independent formulations (tests/formulations.py), never against itself.

Each pin is chosen so that a plausible slip in the oracle fails it:
  * decay applied after instead of before the delta write  -> hand-worked
    T=2 case, matrix and dense formulations;
  * output read from S_{t-1} instead of S_t                -> hand-worked case,
    causal linear attention case;
  * transposed state (S q instead of S^T q)                -> causal linear
    attention case (non-symmetric V);
  * missing sigmoid on beta, wrong gate sign or clamp      -> gate closed forms,
    general-beta linear attention case;
  * state not reset between sequences / wrong offsets      -> varlen pins.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from formulations import chunked_sequence, dense_sequence, matrix_recurrence

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RTOL = 1e-12


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def rand_case(seed, T, H=2, K=8, V=6, N=1, init=True, lb=-5.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, T, H, K))
    k = rng.standard_normal((1, T, H, K))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, H, V))
    g = rng.standard_normal((1, T, H, K))
    beta = rng.standard_normal((1, T, H))
    A_log = np.log(rng.uniform(1, 16, size=H))
    dt_bias = 0.1 * rng.standard_normal(H * K)
    S0 = 0.3 * rng.standard_normal((N, H, K, V)) if init else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, A_log=A_log, dt_bias=dt_bias,
                lower_bound=lb, scale=1.0 / math.sqrt(K), initial_state=S0)


def run(c, **over):
    d = dict(c)
    d.update(over)
    return oracle.kda_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"],
                              d["dt_bias"], d["lower_bound"], d["scale"],
                              initial_state=d.get("initial_state"),
                              cu_seqlens=d.get("cu_seqlens"))


# ---------------------------------------------------------------- gate pins
def test_gate_closed_forms():
    # softplus(0) = ln 2 with A = exp(0) = 1 -> a = -ln 2
    a = oracle.gate_log_decay(np.zeros((1, 1)), np.zeros(1), np.zeros(1), -5.0)
    assert abs(a[0, 0] + math.log(2.0)) < 1e-15
    # softplus(ln(e - 1)) = 1, A = exp(ln 2) = 2 -> a = -2
    x = math.log(math.e - 1.0)
    a = oracle.gate_log_decay(np.full((1, 1), x), np.zeros(1), np.array([math.log(2.0)]), -5.0)
    assert abs(a[0, 0] + 2.0) < 1e-14
    # dt_bias enters additively per (head, channel): g + dt_bias = ln(e - 1)
    a = oracle.gate_log_decay(np.array([[0.0, x - 0.25]]), np.array([x, 0.25]), np.zeros(1), -5.0)
    assert np.allclose(a, [[-1.0, -1.0]], atol=1e-14, rtol=0)
    # large pre-activation saturates at the lower bound
    a = oracle.gate_log_decay(np.full((1, 1), 50.0), np.zeros(1), np.zeros(1), -5.0)
    assert a[0, 0] == -5.0
    # A_log = -inf means A = 0: no decay (a = -0, alpha = 1)
    a = oracle.gate_log_decay(np.full((1, 1), 3.0), np.zeros(1), np.array([-np.inf]), -5.0)
    assert a[0, 0] == 0.0 and math.exp(a[0, 0]) == 1.0
    # very negative pre-activation: softplus ~ e^x, decay ~ -A e^x
    a = oracle.gate_log_decay(np.full((1, 1), -30.0), np.zeros(1), np.zeros(1), -5.0)
    assert abs(a[0, 0] + math.exp(-30.0)) < 1e-25
    # per-head A: head 1 decays twice as fast as head 0 (log A differs by ln 2)
    a = oracle.gate_log_decay(np.zeros((2, 1)), np.zeros(2), np.array([0.0, math.log(2.0)]), -5.0)
    assert abs(a[1, 0] - 2 * a[0, 0]) < 1e-15


def test_beta_sigmoid_closed_forms():
    assert oracle.sigmoid(np.array(0.0)) == 0.5
    assert abs(oracle.sigmoid(np.array(math.log(3.0))) - 0.75) < 1e-15
    assert oracle.sigmoid(np.array(np.inf)) == 1.0
    assert oracle.sigmoid(np.array(-np.inf)) == 0.0


# ------------------------------------------------------- hand-worked golden
def test_hand_worked_two_tokens():
    with open(os.path.join(GOLDEN, "hand_worked_T2.json")) as f:
        gold = json.load(f)
    i = gold["inputs"]
    q = np.array(i["q"])[None, :, None, :]
    k = np.array(i["k"])[None, :, None, :]
    v = np.array(i["v"])[None, :, None, :]
    g = np.array(i["g"])[None, :, None, :]
    b = np.array(i["beta_logit"])[None, :, None]
    S0 = np.array(i["initial_state"])[None, None]
    o, fin = oracle.kda_forward(q, k, v, g, b, np.array(i["A_log"]), np.array(i["dt_bias"]),
                                i["lower_bound"], i["scale"], initial_state=S0)
    assert np.allclose(o[0, :, 0, :], gold["expected"]["o"], atol=1e-14, rtol=0)
    assert np.allclose(fin[0, 0], gold["expected"]["final_state"], atol=1e-14, rtol=0)


# ------------------------------------------------ independent formulations
@pytest.mark.parametrize("K,V,T", [(4, 4, 1), (4, 3, 17), (8, 6, 40), (128, 128, 64)])
def test_dense_formulation(K, V, T):
    c = rand_case(11 + T, T, H=2, K=K, V=V)
    o, fin = run(c)
    for h in range(2):
        O, S = dense_sequence(c["q"][0, :, h], c["k"][0, :, h], c["v"][0, :, h], c["g"][0, :, h],
                              c["beta"][0, :, h], c["A_log"][h], c["dt_bias"][h * K:(h + 1) * K],
                              c["lower_bound"], c["scale"], c["initial_state"][0, h])
        assert rel(o[0, :, h], O) < 1e-11
        assert rel(fin[0, h], S) < 1e-11


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 64])
def test_chunked_formulation(chunk):
    T, K, V = 75, 16, 8            # ragged last chunk for every chunk size > 1
    c = rand_case(5, T, H=2, K=K, V=V, lb=-1.0)
    o, fin = run(c)
    for h in range(2):
        O, S = chunked_sequence(c["q"][0, :, h], c["k"][0, :, h], c["v"][0, :, h], c["g"][0, :, h],
                                c["beta"][0, :, h], c["A_log"][h], c["dt_bias"][h * K:(h + 1) * K],
                                c["lower_bound"], c["scale"], c["initial_state"][0, h], chunk)
        assert rel(o[0, :, h], O) < 1e-11
        assert rel(fin[0, h], S) < 1e-11


def test_matrix_recurrence():
    T, K, V = 12, 5, 3
    c = rand_case(3, T, H=1, K=K, V=V)
    o, fin = run(c)
    O, S = matrix_recurrence(c["q"][0, :, 0], c["k"][0, :, 0], c["v"][0, :, 0], c["g"][0, :, 0],
                             c["beta"][0, :, 0], c["A_log"][0], c["dt_bias"], c["lower_bound"],
                             c["scale"], c["initial_state"][0, 0])
    assert rel(o[0, :, 0], O) < 1e-13
    assert rel(fin[0, 0], S) < 1e-13


# -------------------------------------------------------------- closed forms
def test_beta_zero_is_pure_channel_decay():
    T, K, V = 20, 8, 5
    c = rand_case(7, T, H=2, K=K, V=V)
    b0 = np.full_like(c["beta"], -np.inf)
    o, fin = run(c, beta=b0)
    a = oracle.gate_log_decay(c["g"], c["dt_bias"], c["A_log"], c["lower_bound"])[0]   # [T,H,K]
    G = np.cumsum(a, axis=0)
    for h in range(2):
        S0 = c["initial_state"][0, h]
        for t in range(T):
            St = np.exp(G[t, h])[:, None] * S0
            assert np.allclose(o[0, t, h], c["scale"] * St.T @ c["q"][0, t, h], rtol=1e-12, atol=1e-15)
        assert np.allclose(fin[0, h], np.exp(G[-1, h])[:, None] * S0, rtol=1e-12, atol=1e-15)
    o, fin = run(c, beta=b0, initial_state=None)
    assert np.all(o == 0.0) and np.all(fin == 0.0)


def test_no_decay_no_write_freezes_state():
    T, K, V = 9, 6, 4
    c = rand_case(8, T, H=2, K=K, V=V)
    o, fin = run(c, beta=np.full_like(c["beta"], -np.inf), A_log=np.full(2, -np.inf))
    for h in range(2):
        S0 = c["initial_state"][0, h]
        assert np.allclose(o[0, :, h], c["scale"] * c["q"][0, :, h] @ S0, rtol=1e-13, atol=0)
        assert np.array_equal(fin[0, h], S0)


@pytest.mark.parametrize("general_beta", [False, True])
def test_orthonormal_keys_give_causal_linear_attention(general_beta):
    T, K, V = 24, 32, 7
    rng = np.random.default_rng(21)
    c = rand_case(21, T, H=1, K=K, V=V, init=False)
    perm = rng.permutation(K)[:T]
    k = np.zeros((1, T, 1, K))
    k[0, np.arange(T), 0, perm] = 1.0
    bl = rng.standard_normal((1, T, 1)) if general_beta else np.full((1, T, 1), np.inf)
    o, fin = run(c, k=k, beta=bl, A_log=np.array([-np.inf]))
    Q, Kk, Vv = c["q"][0, :, 0], k[0, :, 0], c["v"][0, :, 0]
    beta = 1.0 / (1.0 + np.exp(-bl[0, :, 0]))
    expect = c["scale"] * np.tril(Q @ Kk.T) @ (beta[:, None] * Vv)
    assert np.allclose(o[0, :, 0], expect, rtol=1e-13, atol=1e-15)
    assert np.allclose(fin[0, 0], Kk.T @ (beta[:, None] * Vv), rtol=1e-13, atol=1e-15)


def test_repeated_key_retrieves_latest_value():
    # alpha = 1, beta = 1, one unit key u: every write replaces the value stored
    # along u, so reading with q = u returns v_t exactly (scale = 1).
    T, K, V = 15, 10, 4
    c = rand_case(4, T, H=1, K=K, V=V)
    u = c["k"][0, 0, 0]
    k = np.broadcast_to(u, (1, T, 1, K)).copy()
    o, fin = run(c, k=k, q=k, beta=np.full((1, T, 1), np.inf), A_log=np.array([-np.inf]), scale=1.0)
    assert np.allclose(o[0, :, 0], c["v"][0, :, 0], rtol=0, atol=1e-13)


# ---------------------------------------------------- invariants on states
def _prefix_states(c, T):
    """S_t for t = 0..T (S_0 = initial) from runs on every prefix."""
    states = [c["initial_state"][0]]
    for t in range(1, T + 1):
        sub = {x: c[x][:, :t] for x in ("q", "k", "v", "g", "beta")}
        _, fin = run(c, **sub)
        states.append(fin[0])
    return states


def test_retrieval_identity_every_step():
    T, K, V = 10, 8, 5
    c = rand_case(9, T, H=2, K=K, V=V)
    st = _prefix_states(c, T)
    a = oracle.gate_log_decay(c["g"], c["dt_bias"], c["A_log"], c["lower_bound"])[0]
    beta = 1.0 / (1.0 + np.exp(-c["beta"][0]))
    for t in range(T):
        for h in range(2):
            kt = c["k"][0, t, h]
            DS = np.exp(a[t, h])[:, None] * st[t][h]
            nk = kt @ kt
            lhs = st[t + 1][h].T @ kt
            rhs = (1 - beta[t, h] * nk) * (DS.T @ kt) + beta[t, h] * nk * c["v"][0, t, h]
            assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-14)


def test_frobenius_bound_every_step():
    T, K, V = 12, 8, 5
    c = rand_case(10, T, H=2, K=K, V=V)
    st = _prefix_states(c, T)
    beta = 1.0 / (1.0 + np.exp(-c["beta"][0]))
    for t in range(T):
        for h in range(2):
            lhs = np.linalg.norm(st[t + 1][h])
            rhs = np.linalg.norm(st[t][h]) + beta[t, h] * np.linalg.norm(c["v"][0, t, h])
            assert lhs <= rhs * (1 + 1e-12)


def test_split_invariance():
    T, K, V = 50, 8, 6
    c = rand_case(12, T, H=3, K=K, V=V)
    o, fin = run(c)
    for t1 in (1, 17, 32, 49):
        a = {x: c[x][:, :t1] for x in ("q", "k", "v", "g", "beta")}
        b = {x: c[x][:, t1:] for x in ("q", "k", "v", "g", "beta")}
        o1, f1 = run(c, **a)
        o2, f2 = run(c, **b, initial_state=f1)
        assert rel(np.concatenate([o1, o2], axis=1), o) < 1e-13
        assert rel(f2, fin) < 1e-13


def test_varlen_equals_independent_runs():
    lens = [5, 0, 13, 1, 21]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    K, V, H = 8, 6, 2
    c = rand_case(13, T, H=H, K=K, V=V, N=len(lens))
    o, fin = run(c, cu_seqlens=cu)
    for n, L in enumerate(lens):
        s, e = cu[n], cu[n + 1]
        sub = {x: c[x][:, s:e] for x in ("q", "k", "v", "g", "beta")}
        on, fn = run(c, **sub, initial_state=c["initial_state"][n:n + 1])
        assert np.array_equal(o[:, s:e], on)
        assert np.array_equal(fin[n], fn[0])
    # a zero-length sequence hands its initial state straight through
    assert np.array_equal(fin[1], c["initial_state"][1])


def test_fixed_batch_equals_packed_varlen():
    B, T, K, V, H = 3, 11, 8, 4, 2
    rng = np.random.default_rng(14)
    c = rand_case(14, B * T, H=H, K=K, V=V, N=B)
    batched = {x: c[x].reshape((B, T) + c[x].shape[2:]) for x in ("q", "k", "v", "g", "beta")}
    o_b, f_b = run(c, **batched)
    cu = np.arange(0, B * T + 1, T, dtype=np.int32)
    o_v, f_v = run(c, cu_seqlens=cu)
    assert np.array_equal(o_b.reshape(o_v.shape), o_v)
    assert np.array_equal(f_b, f_v)
    del rng


# ------------------------------------------------------ numpy vs C oracle
def test_c_oracle_matches_numpy_tiny_workload():
    inp = kda_inputs.generate(kda_inputs.WORKLOADS["tiny_T256_H2"])
    o1, f1 = oracle.numpy_forward(inp)
    o2, f2 = oracle.cref_forward(inp)
    assert rel(o2, o1) < 1e-12 and rel(f2, f1) < 1e-12


def test_c_oracle_matches_numpy_varlen_with_state():
    inp = kda_inputs.random_small(31, B=1, T=150, H=3, seq_lens=[40, 0, 77, 33],
                                  initial_state=True)
    o1, f1 = oracle.numpy_forward(inp)
    o2, f2 = oracle.cref_forward(inp)
    assert rel(o2, o1) < 1e-12 and rel(f2, f1) < 1e-12
    # head subset returns exactly those heads
    o3, f3 = oracle.cref_forward(inp, heads=[2, 0])
    assert np.array_equal(o3[:, :, 0], o2[:, :, 2]) and np.array_equal(f3[:, 1], f2[:, 0])


def test_c_oracle_matches_numpy_batched_fp32_state():
    inp = kda_inputs.random_small(32, B=2, T=40, H=2, initial_state=True)
    inp["initial_state"] = inp["initial_state"].to(torch.float32) * 3.0
    o1, f1 = oracle.numpy_forward(inp)
    o2, f2 = oracle.cref_forward(inp)
    assert rel(o2, o1) < 1e-12 and rel(f2, f1) < 1e-12


def test_c_oracle_truncated_headline_shape():
    # full head dimension and head count of the T=8192, H=96 workload,
    # truncated in time so numpy finishes quickly
    w = kda_inputs.custom("trunc", seed=2, B=1, T=96, H=96, initial_state=True)
    inp = kda_inputs.generate(w)
    o1, f1 = oracle.numpy_forward(inp)
    o2, f2 = oracle.cref_forward(inp)
    assert rel(o2, o1) < 1e-12 and rel(f2, f1) < 1e-12


# -------------------------------------------------------- input generator
def test_generator_is_seeded_and_shaped():
    w = kda_inputs.WORKLOADS["tiny_T256_H2"]
    a, b = kda_inputs.generate(w), kda_inputs.generate(w)
    for key in ("q", "k", "v", "g", "beta", "A_log", "dt_bias"):
        assert torch.equal(a[key], b[key])
    assert a["q"].dtype == torch.bfloat16 and a["q"].shape == (1, 256, 2, 128)
    n = torch.linalg.vector_norm(a["k"].float(), dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-2)
    assert float(a["A_log"].min()) >= 0.0 and float(a["A_log"].max()) <= math.log(16.0)


def test_mixed_lengths_recipe():
    lens = kda_inputs.mixed_lengths(4)
    assert len(lens) == 12 and sum(lens) == 8192
    assert all(64 <= x <= 4096 for x in lens)
    assert kda_inputs.mixed_lengths(4) == lens


def test_varlen_without_initial_state_resets_to_zero():
    lens = [7, 12, 0, 9]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    c = rand_case(15, T, H=2, K=8, V=5, init=False)
    o, fin = run(c, cu_seqlens=cu)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        sub = {x: c[x][:, s:e] for x in ("q", "k", "v", "g", "beta")}
        on, fn = run(c, **sub)
        assert np.array_equal(o[:, s:e], on)
        assert np.array_equal(fin[n], fn[0])
    assert np.all(fin[2] == 0.0)
    # the C oracle agrees on the same packed batch
    inp = kda_inputs.random_small(16, B=1, T=60, H=2, seq_lens=[20, 25, 15])
    o1, f1 = oracle.numpy_forward(inp)
    o2, f2 = oracle.cref_forward(inp)
    assert rel(o2, o1) < 1e-12 and rel(f2, f1) < 1e-12
