"""Codec of the 32-token hand-off record (K = V = 64 or 128), test helper.

A record holds one (32-token chunk, head) in the register layouts of the
scan's 16x16x32 bf16 MFMA operands; lane l of a wave holds row l % 16 of a
16-row tile and 8 consecutive k values starting at 8 (l / 16):
  bytes     0 ..  8191  Kt  [kb 0..3][rt 0..1][lane][8 bf16]:
                        Kt[16 rt + l%16][32 kb + 8 (l/16) + i]
  bytes  8192 .. 16383  Qt  the same for Qt
  bytes 16384 .. 24575  W^T [t 0..7][lane][8 bf16]:
                        W[tau(8 (l/16) + i)][state_chan(t, l%16)]
  bytes 24576 .. 26623  M   [rt 0..1][lane][8 bf16]:
                        M[16 rt + l%16][tau(8 (l/16) + i)]
  bytes 26624 .. 27135  gamma, 128 fp32 (chunk decay per key channel)
  bytes 27136 .. 27647  unused
with tau the token order in which the scan's accumulators hold the rows of
X and state_chan the state-row order of its accumulator tiles.  K = 64 uses
the same layout with the channels from 64 on zero.
"""
from __future__ import annotations

import numpy as np
import torch

REC = 27648
CS = 32


def state_chan(t, rho):
    return 32 * (t // 2) + 8 * (rho // 4) + 4 * (t % 2) + rho % 4


def tau(kappa):
    """Token of k index kappa in the W^T and M operands."""
    g, i = kappa // 8, kappa % 8
    return 4 * g + i if i < 4 else 16 + 4 * g + i - 4


def bf16_words_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16_words(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (nearest even, as the GPU's conversion) -> uint16 words."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    return bf16_words_to_f64(to_bf16_words(x)).reshape(np.shape(x))


def decode(rec: np.ndarray):
    """One 27648-byte record -> (Kt, Qt, W, M, gamma) in natural layout."""
    u16 = rec.view(np.uint16)
    kt = bf16_words_to_f64(u16[0:4096]).reshape(4, 2, 64, 8)
    qt = bf16_words_to_f64(u16[4096:8192]).reshape(4, 2, 64, 8)
    wt = bf16_words_to_f64(u16[8192:12288]).reshape(8, 64, 8)
    mm = bf16_words_to_f64(u16[12288:13312]).reshape(2, 64, 8)
    Kt = np.zeros((CS, 128)); Qt = np.zeros((CS, 128)); W = np.zeros((CS, 128))
    M = np.zeros((CS, CS))
    for l in range(64):
        r, grp = l % 16, l // 16
        for kb in range(4):
            for rt in range(2):
                Kt[16 * rt + r, 32 * kb + 8 * grp: 32 * kb + 8 * grp + 8] = kt[kb, rt, l]
                Qt[16 * rt + r, 32 * kb + 8 * grp: 32 * kb + 8 * grp + 8] = qt[kb, rt, l]
        for i in range(8):
            tok = tau(8 * grp + i)
            for t in range(8):
                W[tok, state_chan(t, r)] = wt[t, l, i]
            for rt in range(2):
                M[16 * rt + r, tok] = mm[rt, l, i]
    gam = rec[26624:27136].view(np.float32).astype(np.float64)
    return Kt, Qt, W, M, gam


def encode(Kt, Qt, W, M, gam) -> np.ndarray:
    """(Kt, Qt, W [32 x 128], M [32 x 32], gamma [128]) -> one record; the
    matrices are rounded to bf16, gamma to fp32."""
    kt = np.zeros((4, 2, 64, 8)); qt = np.zeros((4, 2, 64, 8))
    wt = np.zeros((8, 64, 8)); mm = np.zeros((2, 64, 8))
    for l in range(64):
        r, grp = l % 16, l // 16
        for kb in range(4):
            for rt in range(2):
                kt[kb, rt, l] = Kt[16 * rt + r, 32 * kb + 8 * grp: 32 * kb + 8 * grp + 8]
                qt[kb, rt, l] = Qt[16 * rt + r, 32 * kb + 8 * grp: 32 * kb + 8 * grp + 8]
        for i in range(8):
            tok = tau(8 * grp + i)
            for t in range(8):
                wt[t, l, i] = W[tok, state_chan(t, r)]
            for rt in range(2):
                mm[rt, l, i] = M[16 * rt + r, tok]
    rec = np.zeros(REC, dtype=np.uint8)
    u16 = rec.view(np.uint16)
    u16[0:4096] = to_bf16_words(kt.ravel())
    u16[4096:8192] = to_bf16_words(qt.ravel())
    u16[8192:12288] = to_bf16_words(wt.ravel())
    u16[12288:13312] = to_bf16_words(mm.ravel())
    rec[26624:27136] = np.asarray(gam, dtype=np.float32).view(np.uint8)
    return rec
