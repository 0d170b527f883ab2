"""Helpers for GPU parity tests: run libkda through the C-ABI binding and
compare with the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import kimi_delta_attention_04_amd as kda

# Tolerances of the parity bar: relative L2 error and max-abs error against
# the fp64 oracle, on o and on the final state separately.
REL_L2_TOL = 5e-3
MAX_ABS_TOL = 3e-2


def to_device(inp: dict, device="cuda") -> dict:
    out = {}
    for key, val in inp.items():
        out[key] = val.to(device) if isinstance(val, torch.Tensor) else val
    return out


def run_kda(dinp: dict, final_dtype=torch.float32, poison=True, want_final=True,
            initial_state="from_inputs"):
    """Run kda.fwd on device inputs; outputs are NaN-poisoned first so any
    element the kernels fail to write shows up."""
    q = dinp["q"]
    B, T, H, _ = q.shape
    V = dinp["v"].shape[-1]
    cu = dinp.get("cu_seqlens")
    N = B if cu is None else cu.numel() - 1
    fill = float("nan") if poison else 0.0
    out = torch.full((B, T, H, V), fill, dtype=torch.bfloat16, device=q.device)
    fin = None
    if want_final:
        fin = torch.full((N, H, q.shape[-1], V), fill, dtype=final_dtype, device=q.device)
    init = dinp.get("initial_state") if initial_state == "from_inputs" else initial_state
    kda.fwd(q, dinp["k"], dinp["v"], dinp["g"], dinp["beta"], dinp["scale"], out,
            dinp["A_log"], dinp.get("dt_bias"), dinp["lower_bound"],
            initial_state=init, final_state=fin, cu_seqlens=cu)
    torch.cuda.synchronize()
    return out, fin


# A reference whose norm lies below the fp32 range (state decayed to nothing
# in fp64) counts as zero: only the max-abs bar applies to it.
ZERO_NORM = 1e-30


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.linalg.norm(x - ref)
    n = np.linalg.norm(ref)
    return float(d / n) if n > ZERO_NORM else 0.0


def max_abs(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref))) if x.size else 0.0


def assert_close(name, x, ref, rel_tol=REL_L2_TOL, abs_tol=MAX_ABS_TOL):
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x)), f"{name}: non-finite values (unwritten or overflow)"
    r, m = rel_l2(x, ref), max_abs(x, ref)
    assert r <= rel_tol and m <= abs_tol, f"{name}: rel_l2={r:.3e} (tol {rel_tol}) max_abs={m:.3e} (tol {abs_tol})"
    return r, m


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()
