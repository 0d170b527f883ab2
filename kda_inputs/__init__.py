"""Seeded synthetic inputs for the KDA chunked forward pass.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no gate, no decay, no recurrence), so both the CPU oracle
and the HIP path may consume what it produces.

The workloads mirror the ones the FlashKDA write-ups benchmark on (sequence
length 8192, head dimension 128, 64 or 96 heads, fixed length, uniform
variable length 8 x 1024 and mixed variable length; see "Moonshot AI Rilis
FlashKDA", benchmark paragraph, and "Moonshot AI Open-Sources FlashKDA",
section "The performance gap FlashKDA closes"). No public dataset is involved.

Recipe (identical for every workload):
  * torch CPU generator seeded with the workload's seed; fp32 draws in the
    order q, k, v, g, beta, A_log, dt_bias, initial_state;
  * q, k ~ N(0, 1), L2-normalised per (token, head) vector in fp32, then cast
    to bf16 with round-to-nearest-even;
  * v, g, beta logits ~ N(0, 1), cast to bf16;
  * A_log = log(U[1, 16]) per head (fp32), dt_bias ~ N(0, 0.1) per
    (head, channel) (fp32, flat [H*K]);
  * lower_bound = -5, scale = 1/sqrt(K);
  * initial_state, when the workload has one, ~ N(0, 0.02) [N, H, K, V],
    cast to bf16;
  * mixed variable length: 12 sequence lengths drawn by seeded rejection
    sampling (numpy default_rng(seed)): 11 lengths round(exp(U(ln 64,
    ln 4096))), the 12th takes the remainder of the 8192 tokens and the draw
    is accepted only if that remainder also lies in [64, 4096].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    T: int            # tokens per batch row (packed total when varlen)
    H: int
    K: int = HEAD_DIM
    V: int = HEAD_DIM
    seq_lens: Optional[tuple] = None   # varlen: lengths packed along T (B == 1)
    initial_state: bool = False        # bf16 N(0, 0.02) initial state per sequence
    lower_bound: float = -5.0

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens) if self.seq_lens is not None else self.B

    @property
    def cu_seqlens(self) -> Optional[list]:
        if self.seq_lens is None:
            return None
        cu = [0]
        for n in self.seq_lens:
            cu.append(cu[-1] + int(n))
        return cu

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def describe(self) -> dict:
        d = {"workload": self.name, "B": self.B, "T": self.T, "H": self.H,
             "K": self.K, "V": self.V, "seed": self.seed,
             "initial_state": "bf16" if self.initial_state else None,
             "final_state": "fp32", "lower_bound": self.lower_bound}
        if self.seq_lens is not None:
            d["cu_seqlens"] = self.cu_seqlens
        return d


def mixed_lengths(seed: int, total: int = 8192, count: int = 12,
                  lo: int = 64, hi: int = 4096) -> tuple:
    """Seeded log-uniform lengths on [lo, hi] whose sum is `total`.

    Plain "draw 12 and let the last absorb the remainder" is infeasible on
    average (11 draws already exceed 8192), so draws are rejected until the
    remainder itself lies in [lo, hi].
    """
    rng = np.random.default_rng(seed)
    for _ in range(100000):
        draw = np.round(np.exp(rng.uniform(math.log(lo), math.log(hi), size=count - 1)))
        draw = draw.astype(np.int64)
        rem = total - int(draw.sum())
        if lo <= rem <= hi:
            return tuple(int(x) for x in draw) + (rem,)
    raise RuntimeError("rejection sampling did not converge")


def uniform_lengths(count: int, length: int) -> tuple:
    return tuple([length] * count)


# The five workloads: a tiny one the oracle finishes instantly, then the
# T=8192 / D=128 shapes of the write-ups (64 and 96 heads; fixed, uniform
# varlen 8 x 1024, mixed varlen with 12 sequences).
WORKLOADS = {
    "tiny_T256_H2": Workload("tiny_T256_H2", seed=0, B=1, T=256, H=2),
    "fixed_T8192_H64": Workload("fixed_T8192_H64", seed=1, B=1, T=8192, H=64),
    "fixed_T8192_H96": Workload("fixed_T8192_H96", seed=2, B=1, T=8192, H=96,
                                initial_state=True),
    "varlen_uniform_8x1024_H96": Workload("varlen_uniform_8x1024_H96", seed=3, B=1,
                                          T=8192, H=96,
                                          seq_lens=uniform_lengths(8, 1024)),
    "varlen_mixed12_H96": Workload("varlen_mixed12_H96", seed=4, B=1, T=8192, H=96,
                                   seq_lens=mixed_lengths(4), initial_state=True),
    "varlen_mixed12_H64": Workload("varlen_mixed12_H64", seed=4, B=1, T=8192, H=64,
                                   seq_lens=mixed_lengths(4), initial_state=True),
}

HEADLINE = "fixed_T8192_H96"
# The T = 8192 workloads a benchmark run times (the headline first).
BENCH_WORKLOADS = ("fixed_T8192_H96", "fixed_T8192_H64", "varlen_uniform_8x1024_H96",
                   "varlen_mixed12_H96", "varlen_mixed12_H64")


def custom(name: str, seed: int, B: int, T: int, H: int, seq_lens=None,
           initial_state: bool = False, lower_bound: float = -5.0) -> Workload:
    return Workload(name, seed=seed, B=B, T=T, H=H,
                    seq_lens=tuple(seq_lens) if seq_lens is not None else None,
                    initial_state=initial_state, lower_bound=lower_bound)


def _l2norm(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def generate(w: Workload) -> dict:
    """Draw the workload's tensors on the CPU.

    Returns a dict of CPU tensors: q, k, v, g (bf16 [B,T,H,K|V]), beta (bf16
    [B,T,H]), A_log (fp32 [H]), dt_bias (fp32 [H*K]), initial_state (bf16
    [N,H,K,V] or None), cu_seqlens (int32 [N+1] or None) and the scalars
    scale and lower_bound.
    """
    if w.seq_lens is not None:
        assert w.B == 1 and sum(w.seq_lens) == w.T
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    shp = (w.B, w.T, w.H)
    q = _l2norm(torch.randn(*shp, w.K, generator=gen)).to(torch.bfloat16)
    k = _l2norm(torch.randn(*shp, w.K, generator=gen)).to(torch.bfloat16)
    v = torch.randn(*shp, w.V, generator=gen).to(torch.bfloat16)
    g = torch.randn(*shp, w.K, generator=gen).to(torch.bfloat16)
    beta = torch.randn(*shp, generator=gen).to(torch.bfloat16)
    A_log = torch.log(torch.rand(w.H, generator=gen) * 15.0 + 1.0)
    dt_bias = torch.randn(w.H * w.K, generator=gen) * 0.1
    init = None
    if w.initial_state:
        init = (torch.randn(w.num_seqs, w.H, w.K, w.V, generator=gen) * 0.02).to(torch.bfloat16)
    cu = None
    if w.seq_lens is not None:
        cu = torch.tensor(w.cu_seqlens, dtype=torch.int32)
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "A_log": A_log,
            "dt_bias": dt_bias, "initial_state": init, "cu_seqlens": cu,
            "scale": 1.0 / math.sqrt(w.K), "lower_bound": float(w.lower_bound)}


def random_small(seed: int, B: int, T: int, H: int, K: int = 128, V: int = 128,
                 seq_lens=None, initial_state: bool = False,
                 lower_bound: float = -5.0) -> dict:
    """Same recipe at arbitrary small shapes (used by parity and edge tests)."""
    w = Workload("custom", seed=seed, B=B, T=T, H=H, K=K, V=V,
                 seq_lens=tuple(seq_lens) if seq_lens is not None else None,
                 initial_state=initial_state, lower_bound=lower_bound)
    d = generate(w)
    d["workload"] = w
    return d


def output_grads(seed: int, B: int, T: int, H: int, V: int = HEAD_DIM, N: Optional[int] = None,
                 K: int = HEAD_DIM, final: bool = True) -> tuple:
    """Seeded incoming gradients for the backward pass: d_out ~ N(0, 1) cast
    to bf16 [B, T, H, V] and, when `final`, d_final ~ N(0, 0.1) fp32
    [N, H, K, V] (N defaults to B); drawn in that order from a torch CPU
    generator seeded with `seed`."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    d_out = torch.randn(B, T, H, V, generator=gen).to(torch.bfloat16)
    d_final = None
    if final:
        d_final = torch.randn(B if N is None else N, H, K, V, generator=gen) * 0.1
    return d_out, d_final
