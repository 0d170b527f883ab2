"""kda_fwd_noalloc (the entry point for callers that cannot allocate: its
workspace is a fixed device array of the library) against kda_fwd on the
same inputs: bitwise equal outputs and final states (same kernels), and
within the parity bar of the fp64 oracle, on two calls in a row, the second
smaller than the first; sizes whose workspace exceeds the array are
rejected before any launch."""
from __future__ import annotations

import pytest
import torch

import kda_inputs
import kimi_delta_attention_04_amd as kda
import oracle
from gpu_util import assert_close, np64, to_device

pytestmark = pytest.mark.gpu


def run(entry, d, fin_dtype=torch.float32):
    q = d["q"]
    B, T, H, K = q.shape
    cu = d.get("cu_seqlens")
    N = B if cu is None else cu.numel() - 1
    out = torch.full((B, T, H, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((N, H, K, K), float("nan"), dtype=fin_dtype, device="cuda")
    entry(q, d["k"], d["v"], d["g"], d["beta"], d["scale"], out, d["A_log"], d.get("dt_bias"),
          d["lower_bound"], initial_state=d.get("initial_state"), final_state=fin, cu_seqlens=cu)
    torch.cuda.synchronize()
    return out, fin


def test_noalloc_matches_fwd_twice_second_smaller():
    kda.load()
    cases = [
        kda_inputs.random_small(1301, B=1, T=1000, H=16, initial_state=True),
        kda_inputs.random_small(1302, B=1, T=300, H=2, seq_lens=(0, 33, 1, 200, 66),
                                initial_state=True),
    ]
    sizes = []
    for inp in cases:
        B, T, H, K = inp["q"].shape
        N = B if inp.get("cu_seqlens") is None else inp["cu_seqlens"].numel() - 1
        sizes.append(kda.workspace_size(B, T, H, N, K))
        assert sizes[-1] <= kda.NOALLOC_WORKSPACE_BYTES
        d = to_device(inp)
        out_n, fin_n = run(kda.fwd_noalloc, d)
        out_r, fin_r = run(kda.fwd, d)
        assert torch.equal(out_n, out_r)
        assert torch.equal(fin_n, fin_r)
        o_ref, f_ref = oracle.cref_forward(inp)
        assert_close("o", np64(out_n), o_ref)
        assert_close("final_state", np64(fin_n), f_ref)
    assert sizes[1] < sizes[0]


def test_noalloc_rejects_workspace_beyond_the_array():
    """8 sequences x 96 heads (768 (sequence, head) units) take the
    two-kernel path, whose records exceed the array."""
    kda.load()
    T, H = 8192, 96
    lens = (1024,) * 8
    assert kda.workspace_size(1, T, H, len(lens)) > kda.NOALLOC_WORKSPACE_BYTES
    inp = kda_inputs.random_small(1303, B=1, T=T, H=H, seq_lens=lens)
    d = to_device(inp)
    out = torch.empty_like(d["v"])
    with pytest.raises(kda.KDAError) as err:
        kda.fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], out, d["A_log"],
                        d["dt_bias"], d["lower_bound"], cu_seqlens=d["cu_seqlens"])
    assert err.value.status == 2            # KDA_ERR_UNSUPPORTED
