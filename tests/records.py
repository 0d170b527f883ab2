"""Codec of the 16-token hand-off record, test helper.

A record holds one (16-token chunk, head) for KT key channels (the head
dimension: 64, 128 or 256) in the register layouts of the scan's MFMA
operands; lane l of a wave holds row l % 16:
  KT  [kb 0..KT/32-1][lane][8 bf16]  Kt[l%16][32 kb + 8 (l/16) + i]
  QT  the same for Qt                                       (at 32 KT bytes)
  WT  [tp 0..KT/32-1][lane][8 bf16]  W[4 (l/16) + j][state_chan(2 tp + h, l%16)]
      at bf16 4 h + j (two 16x16x16 A operands, tiles 2tp and 2tp+1)
                                                            (at 64 KT bytes)
  M   [lane][4 bf16]                 M[l%16][4 (l/16) + j]  (at 96 KT bytes)
  GAM [KT fp32]                      chunk decay per key channel (512 bytes on)
and the whole padded to a multiple of 1 KB (7168 bytes at KT = 64, 13312 at
128, 26624 at 256).  state_chan is the state-row order of the scan's accumulator
tiles.
"""
from __future__ import annotations

import numpy as np
import torch

CS = 16


def rec_bytes(KT=128):
    return (96 * KT + 512 + 4 * KT + 1023) // 1024 * 1024


REC = rec_bytes(128)


def state_chan(t, rho):
    return 32 * (t // 2) + 8 * (rho // 4) + 4 * (t % 2) + rho % 4


def bf16_words_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16_words(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (nearest even, as the GPU's conversion) -> uint16 words."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    return bf16_words_to_f64(to_bf16_words(x)).reshape(np.shape(x))


def _offsets(KT):
    q = 32 * KT                     # bytes of one 16 x KT bf16 operand
    return 0, q, 2 * q, 3 * q, 3 * q + 512


def decode(rec: np.ndarray, KT=128):
    """One record -> (Kt, Qt, W [16, KT], M [16, 16], gamma [KT])."""
    o_kt, o_qt, o_wt, o_m, o_g = _offsets(KT)
    nkb = KT // 32
    u16 = rec.view(np.uint16)
    kt = bf16_words_to_f64(u16[o_kt // 2:o_qt // 2]).reshape(nkb, 64, 8)
    qt = bf16_words_to_f64(u16[o_qt // 2:o_wt // 2]).reshape(nkb, 64, 8)
    wt = bf16_words_to_f64(u16[o_wt // 2:o_m // 2]).reshape(nkb, 64, 8)
    mm = bf16_words_to_f64(u16[o_m // 2:o_g // 2]).reshape(64, 4)
    Kt = np.zeros((CS, KT)); Qt = np.zeros((CS, KT)); W = np.zeros((CS, KT))
    M = np.zeros((CS, CS))
    for l in range(64):
        r, grp = l % 16, l // 16
        for kb in range(nkb):
            Kt[r, 32 * kb + 8 * grp: 32 * kb + 8 * grp + 8] = kt[kb, l]
            Qt[r, 32 * kb + 8 * grp: 32 * kb + 8 * grp + 8] = qt[kb, l]
            for h in range(2):
                W[4 * grp: 4 * grp + 4, state_chan(2 * kb + h, r)] = wt[kb, l, 4 * h: 4 * h + 4]
        M[r, 4 * grp: 4 * grp + 4] = mm[l]
    gam = rec[o_g:o_g + 4 * KT].view(np.float32).astype(np.float64)
    return Kt, Qt, W, M, gam


def encode(Kt, Qt, W, M, gam, KT=128) -> np.ndarray:
    """(Kt, Qt, W [16, KT], M [16, 16], gamma [KT]) -> one record; the
    matrices are rounded to bf16, gamma to fp32."""
    o_kt, o_qt, o_wt, o_m, o_g = _offsets(KT)
    nkb = KT // 32
    kt = np.zeros((nkb, 64, 8)); qt = np.zeros((nkb, 64, 8)); wt = np.zeros((nkb, 64, 8))
    mm = np.zeros((64, 4))
    for l in range(64):
        r, grp = l % 16, l // 16
        for kb in range(nkb):
            kt[kb, l] = Kt[r, 32 * kb + 8 * grp: 32 * kb + 8 * grp + 8]
            qt[kb, l] = Qt[r, 32 * kb + 8 * grp: 32 * kb + 8 * grp + 8]
            for h in range(2):
                wt[kb, l, 4 * h: 4 * h + 4] = W[4 * grp: 4 * grp + 4, state_chan(2 * kb + h, r)]
        mm[l] = M[r, 4 * grp: 4 * grp + 4]
    rec = np.zeros(rec_bytes(KT), dtype=np.uint8)
    u16 = rec.view(np.uint16)
    u16[o_kt // 2:o_qt // 2] = to_bf16_words(kt.ravel())
    u16[o_qt // 2:o_wt // 2] = to_bf16_words(qt.ravel())
    u16[o_wt // 2:o_m // 2] = to_bf16_words(wt.ravel())
    u16[o_m // 2:o_g // 2] = to_bf16_words(mm.ravel())
    rec[o_g:o_g + 4 * KT] = np.asarray(gam, dtype=np.float32).view(np.uint8)
    return rec
