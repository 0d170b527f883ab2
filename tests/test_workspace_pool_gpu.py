"""The library's workspace pool keeps freed workspace for later calls up to
1 GiB per device, returns what lies above when a stream synchronises, and
kda_trim_workspace returns the rest (reserved memory read back with
kda_workspace_reserved, i.e. the pool's hipMemPoolAttrReservedMemCurrent)."""
from __future__ import annotations

import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
from gpu_util import to_device

pytestmark = pytest.mark.gpu

KEEP = 1 << 30


def test_reserved_memory_is_bounded_and_trimmed():
    kda.load()
    T, H = 4096, 96
    inp = kda_inputs.random_small(1201, B=1, T=T, H=H, initial_state=True)
    d = to_device(inp)
    q = d["q"]
    # a forward's workspace (under 1 GiB) stays reserved for the next call
    out = torch.empty_like(d["v"])
    kda.fwd(q, d["k"], d["v"], d["g"], d["beta"], d["scale"], out, d["A_log"], d["dt_bias"],
            d["lower_bound"], initial_state=d["initial_state"])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    ws = kda.workspace_size(1, T, H, 1)
    kept = kda.workspace_reserved()
    print(f"reserved after a forward: {kept / 2**20:.1f} MiB (workspace {ws / 2**20:.1f} MiB)", flush=True)
    assert ws <= kept <= KEEP
    kda.trim_workspace(0)
    assert kda.workspace_reserved() == 0
    # a backward takes several GB; after a synchronisation at most 1 GiB stays
    d_out, d_final = kda_inputs.output_grads(1202, 1, T, H)
    bf = torch.bfloat16
    dq, dk, dg = (torch.empty_like(q) for _ in range(3))
    dv = torch.empty_like(d["v"])
    dbeta = torch.empty(1, T, H, dtype=bf, device="cuda")
    dA = torch.empty(H, device="cuda")
    kda.bwd(q, d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"], d["dt_bias"],
            d["lower_bound"], d_out.cuda(), dq, dk, dv, dg, dbeta, dA,
            initial_state=d["initial_state"], d_final_state=d_final.cuda())
    torch.cuda.synchronize()
    after = kda.workspace_reserved()
    print(f"reserved after a backward: {after / 2**20:.1f} MiB", flush=True)
    assert after <= KEEP
    assert torch.isfinite(dq).all().item()
    kda.trim_workspace(0)
    assert kda.workspace_reserved() == 0
