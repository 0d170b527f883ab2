"""The opt-in device check of cu_seqlens contents (KDA_CHECK_CU_SEQLENS=1):
bad contents return KDA_ERR_INVALID_ARG before any compute kernel runs, so
the outputs stay as they were; good contents give the unchecked results bit
for bit.  Every bad case is caught by the check, so no kernel ever sees it."""
from __future__ import annotations

import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
from gpu_util import run_kda, to_device

pytestmark = pytest.mark.gpu

INVALID = 1


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    kda.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


@pytest.fixture
def checked(monkeypatch):
    monkeypatch.setenv("KDA_CHECK_CU_SEQLENS", "1")


def varlen_input():
    return kda_inputs.random_small(1201, B=1, T=100, H=2, seq_lens=(30, 0, 70),
                                   initial_state=True)


@pytest.mark.parametrize("bad", [[0, 30, 20, 100],      # decreasing
                                 [0, 30, 30, 99],       # last entry is not T
                                 [1, 30, 30, 100]])     # first entry is not 0
def test_bad_contents_rejected(checked, bad):
    d = to_device(varlen_input())
    d["cu_seqlens"] = torch.tensor(bad, dtype=torch.int32, device="cuda")
    with pytest.raises(kda.KDAError) as ei:
        run_kda(d)
    assert ei.value.status == INVALID


def test_outputs_untouched_on_rejection(checked):
    d = to_device(varlen_input())
    d["cu_seqlens"] = torch.tensor([0, 30, 20, 100], dtype=torch.int32, device="cuda")
    out = torch.full((1, 100, 2, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((3, 2, 128, 128), float("nan"), device="cuda")
    with pytest.raises(kda.KDAError):
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], out, d["A_log"],
                d["dt_bias"], d["lower_bound"], initial_state=d["initial_state"], final_state=fin,
                cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(fin).all()


def test_good_contents_match_unchecked(checked, monkeypatch):
    d = to_device(varlen_input())
    a = run_kda(d)
    monkeypatch.setenv("KDA_CHECK_CU_SEQLENS", "0")
    b = run_kda(d)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_backward_bad_contents_rejected(checked):
    inp = varlen_input()
    d = to_device(inp)
    d_out, _ = kda_inputs.output_grads(1202, 1, 100, 2, N=3)
    d["cu_seqlens"] = torch.tensor([0, 30, 30, 99], dtype=torch.int32, device="cuda")
    q = d["q"]
    grads = [torch.empty_like(q) for _ in range(4)]
    dbeta = torch.empty(1, 100, 2, dtype=torch.bfloat16, device="cuda")
    dA = torch.empty(2, device="cuda")
    with pytest.raises(kda.KDAError) as ei:
        kda.bwd(q, d["k"], d["v"], d["g"], d["beta"], d["scale"], d["A_log"], d["dt_bias"],
                d["lower_bound"], d_out.cuda(), grads[0], grads[1], grads[2], grads[3], dbeta, dA,
                initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    assert ei.value.status == INVALID
