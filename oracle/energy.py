"""Oracle: token-level block energy and the retained attention mass of a mask.

TEST INFRASTRUCTURE ONLY (see the package docstring). Float64 NumPy.

Source: [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse Attention",
key design 1, Eq. (5): with P the row-softmax attention matrix, the energy of query block r
and key block c is E_rc = (1/B) * sum over queries i of block r and keys j of block c of P_ij.
The page notes that each query-block row of E sums to 1. The retained mass of a mask is the
sum of E over its kept blocks ([SparSTAR] "SparSTAR：为什么视频自回归的稀疏注意力不能跨尺度复用？",
Figures 3 and 4 report this quantity per scale and clip).
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

from .select import BLOCK


def block_energy_rows(q, k, rows: Iterable[int], scale: Optional[float] = None,
                      block: int = BLOCK) -> np.ndarray:
    """Eq. (5) for the listed rows r = (b * H + h) * nQB + i, from the dense softmax over all keys.
    q [B, H, Lq, d], k [B, H, Lk, d] -> E [n, nKB]."""
    bsz, heads, lq, d = q.shape
    lk = k.shape[-2]
    nqb, nkb = -(-lq // block), -(-lk // block)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = list(rows)
    out = np.zeros((len(rows), nkb), dtype=np.float64)
    for n, r in enumerate(rows):
        bh, i = divmod(int(r), nqb)
        b, h = divmod(bh, heads)
        # a partial last block holds fewer tokens; B is then the number it holds (reading)
        qi = np.asarray(q[b, h, i * block:min((i + 1) * block, lq)], dtype=np.float64)
        kk = np.asarray(k[b, h], dtype=np.float64)
        logits = (qi @ kk.T) * scale
        e = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)                     # [queries, Lk]
        per_key = p.sum(axis=0)
        for c in range(nkb):
            out[n, c] = per_key[c * block:min((c + 1) * block, lk)].sum() / qi.shape[0]
    return out


def token_upper_bound(q, k, rows: Iterable[int], budgets: Iterable[int],
                      scale: Optional[float] = None, block: int = BLOCK) -> np.ndarray:
    """Token-wise upper bound of the retained mass ([SparSTAR] "SparSTAR：为什么视频自回归的稀疏
    注意力不能跨尺度复用？", Figure 3 compares per-scale block Top-K against it). Reading: for row r
    with a budget of m_r key tokens (a mask of m_r / 128 blocks keeps m_r tokens per query), the
    mean over the block's queries of the sum of that query's m_r largest probabilities under
    the dense softmax. No mask keeping m_r tokens per query retains more, so a block mask's
    retained mass is at most this value."""
    bsz, heads, lq, d = q.shape
    nqb = -(-lq // block)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows, budgets = list(rows), list(budgets)
    out = np.zeros(len(rows), dtype=np.float64)
    for n, (r, m) in enumerate(zip(rows, budgets)):
        bh, i = divmod(int(r), nqb)
        b, h = divmod(bh, heads)
        qi = np.asarray(q[b, h, i * block:min((i + 1) * block, lq)], dtype=np.float64)
        kk = np.asarray(k[b, h], dtype=np.float64)
        logits = (qi @ kk.T) * scale
        e = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        top = -np.sort(-p, axis=1)[:, :int(m)]
        out[n] = top.sum(axis=1).mean()
    return out


def retained_mass(energy, kept) -> np.ndarray:
    """Sum of the block energies over the kept blocks of each row."""
    energy = np.asarray(energy, dtype=np.float64)
    kept = np.asarray(kept, dtype=bool)
    return np.where(kept, energy, 0.0).sum(axis=-1)
