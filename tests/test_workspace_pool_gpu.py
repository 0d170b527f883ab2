"""The library's workspace pool keeps at most 1 GiB of freed workspace
reserved per device after a synchronisation, and kda_trim_workspace returns
the rest (reserved memory read back with kda_workspace_reserved, i.e. the
pool's hipMemPoolAttrReservedMemCurrent)."""
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
    # a backward at T = 4096, H = 96 takes several GB of workspace
    inp = kda_inputs.random_small(1201, B=1, T=4096, H=96, initial_state=True)
    d = to_device(inp)
    d_out, d_final = kda_inputs.output_grads(1202, 1, 4096, 96)
    bf = torch.bfloat16
    q = d["q"]
    dq, dk, dg = (torch.empty_like(q) for _ in range(3))
    dv = torch.empty_like(d["v"])
    dbeta = torch.empty(1, 4096, 96, dtype=bf, device="cuda")
    dA = torch.empty(96, device="cuda")
    kda.bwd(q, d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"], d["dt_bias"],
            d["lower_bound"], d_out.cuda(), dq, dk, dv, dg, dbeta, dA,
            initial_state=d["initial_state"], d_final_state=d_final.cuda())
    torch.cuda.synchronize()
    reserved = kda.workspace_reserved()
    print(f"reserved after a backward and a synchronisation: {reserved / 2**20:.0f} MiB", flush=True)
    assert 0 < reserved <= KEEP
    kda.trim_workspace(0)
    assert kda.workspace_reserved() == 0
    # the pool still serves calls after a trim
    out = torch.empty_like(d["v"])
    kda.fwd(q, d["k"], d["v"], d["g"], d["beta"], d["scale"], out, d["A_log"], d["dt_bias"],
            d["lower_bound"], initial_state=d["initial_state"])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    assert 0 < kda.workspace_reserved() <= KEEP
    kda.trim_workspace(0)
    assert kda.workspace_reserved() == 0
