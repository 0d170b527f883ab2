"""fp64 CPU oracle for the KDA forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Two
implementations of the same token recurrence:

  * kda_ref.kda_forward  - numpy, vectorised over heads (small sizes);
  * cref_forward         - the C/OpenMP version in kda_ref_cpu.c (full sizes,
                           optionally a subset of heads);
and the exact gradient of that recurrence, kda_ref_bwd.kda_backward (numpy,
reverse-mode through the token steps; numpy_backward below) and its C/OpenMP
restatement kda_ref_backward in kda_ref_cpu.c (cref_backward below, for full
sizes).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .kda_ref import gate_log_decay, kda_forward, sigmoid, softplus  # noqa: F401
from .kda_ref_bwd import kda_backward  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda_ref.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.kda_ref_forward.restype = ctypes.c_int
    lib.kda_ref_forward.argtypes = [P, P, P, P, P, P, P, ctypes.c_double, ctypes.c_double,
                                    P, i32, i32, i32, i32, i32, i32,
                                    P, i32, P, i32, P, P, i32]
    lib.kda_ref_backward.restype = ctypes.c_int
    lib.kda_ref_backward.argtypes = [P, P, P, P, P, P, P, ctypes.c_double, ctypes.c_double,
                                     P, i32, i32, i32, i32, i32, i32, P, i32, P, P,
                                     P, i32, i32, P, P, P, P, P, P, P, P, i32]
    lib.kda_ref_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().kda_ref_max_threads())


def _bits(t) -> np.ndarray:
    """Raw bf16 bit patterns of a CPU bf16 torch tensor as a uint16 array."""
    import torch
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def cref_forward(inp: dict, heads=None, threads: int = 0, want_final: bool = True):
    """Run the C oracle on a generated input dict (see kda_inputs.generate).

    heads: optional list of head indices; outputs then hold only those heads,
    in that order.  Returns (o [B, T, nsel, V] fp64, final [N, nsel, K, V]
    fp64 or None).
    """
    import torch
    lib = _load()
    q, k, v, g, beta = (inp[x] for x in ("q", "k", "v", "g", "beta"))
    B, T, H, K = q.shape
    V = v.shape[-1]
    cu = inp.get("cu_seqlens")
    N = B if cu is None else int(cu.numel()) - 1
    sel = list(range(H)) if heads is None else [int(h) for h in heads]
    nsel = len(sel)
    bq, bk, bv, bg, bb = (_bits(x) for x in (q, k, v, g, beta))
    A_log = inp["A_log"].to(torch.float32).contiguous().numpy()
    dtb = inp.get("dt_bias")
    dtb = None if dtb is None else dtb.to(torch.float32).contiguous().numpy()
    init = inp.get("initial_state")
    init_arr, init_dtype = None, 0
    if init is not None:
        if init.dtype == torch.bfloat16:
            init_arr, init_dtype = _bits(init), 0
        else:
            init_arr, init_dtype = init.to(torch.float32).contiguous().numpy(), 1
    cu_arr = None if cu is None else cu.to(torch.int32).contiguous().numpy()
    heads_arr = np.asarray(sel, dtype=np.int32)
    out = np.zeros((B, T, nsel, V), dtype=np.float64)
    final = np.zeros((N, nsel, K, V), dtype=np.float64) if want_final else None

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    rc = lib.kda_ref_forward(ptr(bq), ptr(bk), ptr(bv), ptr(bg), ptr(bb), ptr(A_log), ptr(dtb),
                             float(inp["lower_bound"]), float(inp["scale"]),
                             ptr(cu_arr), N, B, T, H, K, V,
                             ptr(init_arr), init_dtype, ptr(heads_arr), nsel,
                             ptr(out), ptr(final), int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_ref_forward failed with {rc}")
    return out, final


def cref_backward(inp: dict, d_out, d_final=None, heads=None, threads: int = 0,
                  checkpoint: int = 64):
    """Run the C gradient oracle (kda_ref_backward in kda_ref_cpu.c) on a
    generated input dict: the same gradients as numpy_backward, in the same
    dict layout, at full sizes.

    d_out: bf16 [B, T, H, V] tensor; d_final: fp32 [N, H, K, V] tensor or
    None.  heads: optional list of head indices; every output then holds
    only those heads, in that order.
    """
    import torch
    lib = _load()
    q, k, v, g, beta = (inp[x] for x in ("q", "k", "v", "g", "beta"))
    B, T, H, K = q.shape
    V = v.shape[-1]
    cu = inp.get("cu_seqlens")
    N = B if cu is None else int(cu.numel()) - 1
    sel = list(range(H)) if heads is None else [int(h) for h in heads]
    ns = len(sel)
    bq, bk, bv, bg, bb, bdo = (_bits(x) for x in (q, k, v, g, beta, d_out))
    A_log = inp["A_log"].to(torch.float32).contiguous().numpy()
    dtb = inp.get("dt_bias")
    dtb = None if dtb is None else dtb.to(torch.float32).contiguous().numpy()
    init = inp.get("initial_state")
    init_arr, init_dtype = None, 0
    if init is not None:
        if init.dtype == torch.bfloat16:
            init_arr, init_dtype = _bits(init), 0
        else:
            init_arr, init_dtype = init.to(torch.float32).contiguous().numpy(), 1
    dfin = None if d_final is None else d_final.to(torch.float32).contiguous().numpy()
    cu_arr = None if cu is None else cu.to(torch.int32).contiguous().numpy()
    heads_arr = np.asarray(sel, dtype=np.int32)
    out = dict(dq=np.zeros((B, T, ns, K)), dk=np.zeros((B, T, ns, K)), dg=np.zeros((B, T, ns, K)),
               dv=np.zeros((B, T, ns, V)), dbeta=np.zeros((B, T, ns)), dA_log=np.zeros(ns),
               ddt_bias=np.zeros(ns * K), d_initial_state=np.zeros((N, ns, K, V)))

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    rc = lib.kda_ref_backward(ptr(bq), ptr(bk), ptr(bv), ptr(bg), ptr(bb), ptr(A_log), ptr(dtb),
                              float(inp["lower_bound"]), float(inp["scale"]),
                              ptr(cu_arr), N, B, T, H, K, V, ptr(init_arr), init_dtype,
                              ptr(bdo), ptr(dfin), ptr(heads_arr), ns, int(checkpoint),
                              *(ptr(out[x]) for x in ("dq", "dk", "dv", "dg", "dbeta", "dA_log",
                                                      "ddt_bias", "d_initial_state")),
                              int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_ref_backward failed with {rc}")
    return out


def numpy_forward(inp: dict):
    """Run the numpy oracle on a generated input dict (exact fp64 upcasts)."""
    import torch

    def f64(t):
        return None if t is None else t.to(torch.float64).numpy()

    return kda_forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["g"]),
                       f64(inp["beta"]), f64(inp["A_log"]), f64(inp.get("dt_bias")),
                       float(inp["lower_bound"]), float(inp["scale"]),
                       initial_state=f64(inp.get("initial_state")),
                       cu_seqlens=None if inp.get("cu_seqlens") is None
                       else inp["cu_seqlens"].numpy())


def numpy_backward(inp: dict, d_out, d_final=None, heads=None, checkpoint: int = 64):
    """Run the numpy gradient oracle on a generated input dict.

    d_out: [B, T, H, V] tensor; d_final: [N, H, K, V] tensor or None.
    heads: optional list of head indices (heads are independent); every
    output then holds only those heads, in that order.
    """
    import torch

    def f64(t):
        return None if t is None else t.to(torch.float64).numpy()

    H, K = inp["q"].shape[-2], inp["q"].shape[-1]
    sel = list(range(H)) if heads is None else [int(h) for h in heads]
    tok = lambda t: f64(t)[:, :, sel]
    dtb = inp.get("dt_bias")
    dtb = None if dtb is None else f64(dtb).reshape(H, K)[sel].reshape(-1)
    init = inp.get("initial_state")
    cu = inp.get("cu_seqlens")
    return kda_backward(tok(inp["q"]), tok(inp["k"]), tok(inp["v"]), tok(inp["g"]),
                        f64(inp["beta"])[:, :, sel], f64(inp["A_log"])[sel], dtb,
                        float(inp["lower_bound"]), float(inp["scale"]), tok(d_out),
                        d_final=None if d_final is None else f64(d_final)[:, sel],
                        initial_state=None if init is None else f64(init)[:, sel],
                        cu_seqlens=None if cu is None else cu.numpy(), checkpoint=checkpoint)
