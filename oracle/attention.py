"""Oracle: forward attention restricted to the kept key blocks, and the dense reference.

TEST INFRASTRUCTURE ONLY (see the package docstring). Float64 NumPy.

Sources: [SparSTAR] "SparSTAR：为什么视频自回归的稀疏注意力不能跨尺度复用？", method overview,
FastFlex bullet (attention runs only over the selected blocks, forward only); [CalibAtt]
"Accelerating Text-to-Video Generation with Calibrated Sparse Attention", key design 4 (kept
key-block connections are computed from the current Q, K, V; skipped blocks cost nothing).

Reading: every query token of query block i attends, with softmax(q . k * 1/sqrt(d)), to every
token of every key block kept for row i and to nothing else; there is no causal mask. A row with
no kept block gives O = 0 and lse = -inf. lse is the natural log of the softmax denominator.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np

from .select import BLOCK


def _softmax_weighted(logits: np.ndarray, values: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    den = e.sum(axis=-1, keepdims=True)
    out = (e @ values) / den
    lse = (m + np.log(den))[..., 0]
    return out, lse


def attention_rows(q, k, v, row_ptr, col_idx, rows: Optional[Iterable[int]] = None,
                   scale: Optional[float] = None, block: int = BLOCK):
    """Gather formulation. For every listed CSR row r = (b * H + h) * nQB + i, collect the tokens
    of its kept key blocks, then take a dense softmax over them for the 128 queries of block i.
    q [B, H, Lq, d], k and v [B, H, Lk, d]. Returns (O [n, block, d], lse [n, block]) in float64
    for the n listed rows (all rows if rows is None)."""
    bsz, heads, lq, d = q.shape
    lk = k.shape[-2]
    nqb = -(-lq // block)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if rows is None:
        rows = range(bsz * heads * nqb)
    rows = list(rows)
    out = np.zeros((len(rows), block, d), dtype=np.float64)
    lse = np.full((len(rows), block), -np.inf, dtype=np.float64)
    for n, r in enumerate(rows):
        bh, i = divmod(int(r), nqb)
        b, h = divmod(bh, heads)
        cols = np.asarray(col_idx[int(row_ptr[r]):int(row_ptr[r + 1])], dtype=np.int64)
        if cols.size == 0:
            continue
        # tokens of the kept blocks; a partial last key block contributes the tokens it holds
        tok = (cols[:, None] * block + np.arange(block)[None, :]).reshape(-1)
        tok = tok[tok < lk]
        q0, q1 = i * block, min((i + 1) * block, lq)
        qi = np.asarray(q[b, h, q0:q1], dtype=np.float64)
        kt = np.asarray(k[b, h], dtype=np.float64)[tok]
        vt = np.asarray(v[b, h], dtype=np.float64)[tok]
        out[n, :q1 - q0], lse[n, :q1 - q0] = _softmax_weighted((qi @ kt.T) * scale, vt)
    return out, lse


def attention_masked(q, k, v, kept, scale: Optional[float] = None, block: int = BLOCK):
    """Masked formulation, for small inputs: the full logits matrix over all keys with -inf on
    every token of a key block that is not kept. kept [B, H, nQB, nKB] bool.
    Returns (O [B, H, Lq, d], lse [B, H, Lq]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kept = np.asarray(kept, dtype=bool)
    lq, lk = q.shape[-2], k.shape[-2]
    token_mask = np.repeat(np.repeat(kept, block, axis=-2), block, axis=-1)[..., :lq, :lk]
    logits = np.where(token_mask, (q @ np.swapaxes(k, -1, -2)) * scale, -np.inf)
    m = logits.max(axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    e = np.exp(logits - m)
    den = e.sum(axis=-1, keepdims=True)
    safe = np.where(den > 0, den, 1.0)
    out = np.where(den > 0, (e @ v) / safe, 0.0)
    lse = np.where(den[..., 0] > 0, (m + np.log(safe))[..., 0], -np.inf)
    return out, lse


def attention_dense(q, k, v, scale: Optional[float] = None):
    """Dense softmax attention over every key (all blocks kept). Returns (O, lse) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _softmax_weighted((q @ np.swapaxes(k, -1, -2)) * scale, v)
