"""Oracle: the anchor-row path for spatially repeating heads.

TEST INFRASTRUCTURE ONLY (see the package docstring). Float64 NumPy.

Source: [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse Attention",
key design 3 (spatial repetition) and key design 4 (the repeating-head execution path): a frame
of the video has H spatial rows of W tokens; k equally spaced anchor rows per frame attend to all
keys and values, and every spatial row of the frame takes the output of its nearest anchor row
(the query count drops from H W to k W per frame). The default k is 5.

Readings (the page does not spell them out):
  * "equally spaced" anchors are the centres of k equal bands of the H rows:
    a_j = floor((2 j + 1) H / (2 k)), j = 0 .. k - 1;
  * "nearest" is the smallest |r - a_j|, ties to the lower anchor;
  * a row copies the anchor's output at the same column (position within the row);
  * query tokens after the last frame (padding of the sequence to a block multiple) are not
    part of any frame and attend normally, as their own queries;
  * the log-sum-exp of a broadcast row is its anchor's.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def anchor_rows(rows_per_frame: int, n_anchors: int) -> np.ndarray:
    """Indices of the k anchor rows of a frame of H rows (band centres)."""
    h, k = int(rows_per_frame), int(n_anchors)
    if not 1 <= k <= h:
        raise ValueError("need 1 <= n_anchors <= rows_per_frame")
    return np.array([((2 * j + 1) * h) // (2 * k) for j in range(k)], dtype=np.int64)


def nearest_anchor(rows_per_frame: int, n_anchors: int) -> np.ndarray:
    """For each row r of a frame, the index j of its nearest anchor (ties to the lower j)."""
    a = anchor_rows(rows_per_frame, n_anchors)
    out = np.empty(rows_per_frame, dtype=np.int64)
    for r in range(rows_per_frame):
        best, best_d = 0, abs(r - int(a[0]))
        for j in range(1, a.size):
            d = abs(r - int(a[j]))
            if d < best_d:
                best, best_d = j, d
        out[r] = best
    return out


def anchor_attention(q, k, v, frames: int, rows_per_frame: int, row_width: int,
                     n_anchors: int, scale: Optional[float] = None):
    """q [B, H, Lq, d], k and v [B, H, Lk, d] -> (O [B, H, Lq, d], lse [B, H, Lq]) of the anchor
    path: dense softmax attention for the anchor rows' queries and the trailing queries, then
    every spatial row takes its nearest anchor row's output at the same column."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, heads, lq, d = q.shape
    video = frames * rows_per_frame * row_width
    if video > lq:
        raise ValueError("frames x rows x width exceeds the query length")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    anchors = anchor_rows(rows_per_frame, n_anchors)
    near = nearest_anchor(rows_per_frame, n_anchors)
    out = np.zeros_like(q)
    lse = np.zeros(q.shape[:3])

    def dense(qs, kk, vv):
        logits = (qs @ kk.T) * scale
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        s = e.sum(axis=1, keepdims=True)
        return (e / s) @ vv, (m + np.log(s))[:, 0]

    for b in range(bsz):
        for h in range(heads):
            kk, vv = k[b, h], v[b, h]
            for f in range(frames):
                base = f * rows_per_frame * row_width
                anchor_out = {}
                for j, a in enumerate(anchors):
                    sl = slice(base + a * row_width, base + (a + 1) * row_width)
                    anchor_out[j] = dense(q[b, h, sl], kk, vv)
                for r in range(rows_per_frame):
                    o_r, l_r = anchor_out[int(near[r])]
                    sl = slice(base + r * row_width, base + (r + 1) * row_width)
                    out[b, h, sl] = o_r
                    lse[b, h, sl] = l_r
            if video < lq:
                o_t, l_t = dense(q[b, h, video:], kk, vv)
                out[b, h, video:] = o_t
                lse[b, h, video:] = l_t
    return out, lse
