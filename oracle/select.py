"""Oracle: block partition, pooling, block scores, forced set, Top-K / mass selection, CSR.

TEST INFRASTRUCTURE ONLY (see the package docstring). Float64 NumPy; inputs given as bf16 or
fp32 values are widened exactly.

Sources (page title, then the passage):
  [SparSTAR] "SparSTAR：为什么视频自回归的稀疏注意力不能跨尺度复用？" (pchao.org digest), section
      "方法概览" (method overview) and its bullets on block partition with aggregated scoring,
      clip-aware retention, per-head masks and the decreasing density schedule.
  [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse Attention"
      (papernotes.org), "关键设计" (key designs) item 1, Eq. (5) and the rule stated after it,
      and item 4 (read-only skip list per query block).

Readings where the pages say nothing exact (each is also listed in the design notes):
  * S_ic is the dot product of the pooled query and key means times 1/sqrt(d).
  * Top-K keeps K = min(|C|, ceil(density * |C|)) candidates, C = key blocks not forced.
  * Ordering is (score descending, block index ascending); -0.0 equals +0.0.
  * Mass mode works on the softmax of the pooled scores over all key blocks of the row; forced
    blocks count toward the threshold first; "reaches" means >=, decided in exact fixed point:
    u = floor(p * 2^62), threshold = ceil(tau * 2^62); if all candidates do not reach it, every
    block is kept; tau >= 1 keeps every block.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

BLOCK = 128          # [SparSTAR] method overview: sequences are cut into 128-token blocks
MASS_BITS = 62       # fixed-point scale of the exact mass comparison (reading above)


def n_blocks(length: int, block: int = BLOCK) -> int:
    """[SparSTAR] method overview, block partition: token t of a sequence belongs to block
    t // 128. Reading for lengths that are not a whole number of blocks (the pages only show
    whole blocks): the last block is partial and holds the remaining tokens, so there are
    ceil(L / 128) blocks."""
    if length <= 0:
        raise ValueError(f"length {length} is not positive")
    return -(-length // block)


def block_tokens(i: int, length: int, block: int = BLOCK) -> range:
    """Token positions of block i (the last one may hold fewer than `block`)."""
    return range(i * block, min((i + 1) * block, length))


def pool(x, block: int = BLOCK) -> np.ndarray:
    """[SparSTAR] method overview, block partition bullet: the vectors inside each block are
    averaged. x is [..., L, d]; the result is [..., ceil(L / block), d] in float64; a partial last
    block averages the tokens it holds. Pooling runs separately for every (batch, head) slice,
    never across heads ([SparSTAR] per-head bullet)."""
    x = np.asarray(x, dtype=np.float64)
    length, d = x.shape[-2], x.shape[-1]
    nb = n_blocks(length, block)
    out = np.empty(x.shape[:-2] + (nb, d), dtype=np.float64)
    for i in range(nb):
        t = block_tokens(i, length, block)
        out[..., i, :] = x[..., t.start:t.stop, :].mean(axis=-2)
    return out


def block_scores(qbar, kbar, scale: Optional[float] = None) -> np.ndarray:
    """[SparSTAR] method overview: aggregated query-key compatibility of a query block i and a key
    block c, read as S_ic = (qbar_i . kbar_c) * scale with scale = 1/sqrt(d).
    qbar [..., nQB, d], kbar [..., nKB, d] -> S [..., nQB, nKB]."""
    qbar = np.asarray(qbar, dtype=np.float64)
    kbar = np.asarray(kbar, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(qbar.shape[-1])
    return np.matmul(qbar, np.swapaxes(kbar, -1, -2)) * float(scale)


def forced_blocks(nkb: int, text: Tuple[int, int], extra: Tuple[int, int]) -> np.ndarray:
    """[SparSTAR] method overview, clip-aware retention bullet: text key blocks are always kept
    dense; in the first clip the image-pyramid blocks are kept dense too; in later clips only the
    text blocks. Both segments are contiguous key-block ranges [begin, end); an empty range has
    begin == end. Returns a bool mask [nKB], identical for every head and query block."""
    mask = np.zeros(nkb, dtype=bool)
    spans = []
    for begin, end in (text, extra):
        if not (0 <= begin <= end <= nkb):
            raise ValueError(f"forced range [{begin}, {end}) outside [0, {nkb})")
        if begin < end:
            spans.append((begin, end))
    if len(spans) == 2 and spans[0][0] < spans[1][1] and spans[1][0] < spans[0][1]:
        raise ValueError("forced ranges overlap")
    for begin, end in spans:
        mask[begin:end] = True
    return mask


def topk_budget(density: float, n_candidates: int) -> int:
    """[SparSTAR] decreasing density schedule bullet: a density is the fraction of the remaining
    (non-forced) key blocks kept. Reading: K = min(|C|, ceil(density * |C|)) in float64."""
    if not (0.0 <= density <= 1.0):
        raise ValueError("density must lie in [0, 1]")
    return min(n_candidates, int(math.ceil(density * n_candidates)))


def select_topk(scores, forced: np.ndarray, k: int) -> np.ndarray:
    """[SparSTAR] method overview: forced blocks are kept, and a joint Top-K over all other key
    blocks of the row picks the rest, separately for every head and query block. Order:
    score descending, ties to the lower block index. scores [..., nKB] -> kept bool [..., nKB]."""
    s = np.asarray(scores, dtype=np.float64)
    nkb = s.shape[-1]
    rows = s.reshape(-1, nkb)
    kept = np.zeros(rows.shape, dtype=bool)
    kept[:, forced] = True
    cand = np.flatnonzero(~forced)
    if k < 0 or k > cand.size:
        raise ValueError(f"k={k} outside [0, {cand.size}]")
    if k > 0:
        # a stable sort of the negated scores keeps equal scores in ascending index order;
        # -0.0 and +0.0 compare equal, so they tie as well
        order = np.argsort(-rows[:, cand], axis=1, kind="stable")
        chosen = cand[order[:, :k]]
        np.put_along_axis(kept, chosen, True, axis=1)
    return kept.reshape(s.shape)


def block_softmax(scores) -> np.ndarray:
    """Mass-mode energies: softmax of the block scores over all key blocks of each row. This is
    the pooled stand-in for [CalibAtt] Eq. (5); with no spread of the vectors inside a block it is
    exactly that energy. scores [..., nKB] -> p [..., nKB], each row summing to 1."""
    s = np.asarray(scores, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def mass_units(p) -> np.ndarray:
    """Exact fixed-point masses u = floor(p * 2^62) as uint64 (reading above). Scaling by a power
    of two and flooring are exact in float64 for the values involved."""
    p = np.asarray(p, dtype=np.float64)
    if np.any(p < 0) or np.any(p >= 2.0):
        raise ValueError("energies must lie in [0, 2)")
    return np.floor(p * float(2 ** MASS_BITS)).astype(np.uint64)


def mass_threshold_units(tau: float) -> int:
    """Threshold in the same fixed point: ceil(tau * 2^62)."""
    return int(math.ceil(float(tau) * float(2 ** MASS_BITS)))


def select_mass(p, forced: np.ndarray, tau: float) -> np.ndarray:
    """[CalibAtt] key design 1: per query-block row, sort the key blocks by energy from high to
    low, keep the shortest prefix whose accumulated energy reaches the threshold, and map the
    result back to the original block positions. Here the forced blocks are kept first and count
    toward the threshold; candidates follow in (energy descending, index ascending) order.
    p [..., nKB] -> kept bool [..., nKB]."""
    if not (0.0 < tau <= 1.0):
        raise ValueError("mass threshold must lie in (0, 1]")
    p = np.asarray(p, dtype=np.float64)
    nkb = p.shape[-1]
    rows = p.reshape(-1, nkb)
    kept = np.zeros(rows.shape, dtype=bool)
    if tau >= 1.0:
        kept[:] = True
        return kept.reshape(p.shape)
    kept[:, forced] = True
    theta = mass_threshold_units(tau)
    u = mass_units(rows)
    cand = np.flatnonzero(~forced)
    for r in range(rows.shape[0]):
        have = sum(int(x) for x in u[r, forced])
        if have >= theta:
            continue
        order = cand[np.argsort(-rows[r, cand], kind="stable")]
        acc = have
        reached = False
        for c in order:
            kept[r, c] = True
            acc += int(u[r, c])
            if acc >= theta:
                reached = True
                break
        if not reached:
            kept[r, :] = True
    return kept.reshape(p.shape)


def to_csr(kept) -> Tuple[np.ndarray, np.ndarray]:
    """[CalibAtt] key design 4: for each query block, the key blocks to visit, read-only, forward
    direction only ([SparSTAR] FastFlex bullet: no backward index structures). kept [rows, nKB]
    -> (row_ptr [rows+1] int64, exclusive prefix of the counts; col_idx [nnz] int64, ascending
    within each row)."""
    kept = np.asarray(kept, dtype=bool)
    kept = kept.reshape(-1, kept.shape[-1])
    counts = kept.sum(axis=1)
    row_ptr = np.zeros(kept.shape[0] + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = np.nonzero(kept)[1].astype(np.int64)    # row-major: ascending inside each row
    return row_ptr, col_idx


def to_intervals(kept) -> Tuple[np.ndarray, np.ndarray]:
    """[CalibAtt] key design 4: the skip list stores, per query block, the contiguous runs of
    key blocks it needs. kept [rows, nKB] -> (iv_ptr [rows+1] int64, exclusive prefix of the run
    counts; iv [n_runs, 2] int64 half-open [start, end) block ranges, ascending and maximal
    (two runs of a row never touch))."""
    kept = np.asarray(kept, dtype=bool)
    kept = kept.reshape(-1, kept.shape[-1])
    starts, ptr = [], [0]
    for row in kept:
        padded = np.concatenate([[False], row, [False]]).astype(np.int8)
        edge = np.diff(padded)
        b = np.nonzero(edge == 1)[0]
        e = np.nonzero(edge == -1)[0]
        starts.extend(zip(b.tolist(), e.tolist()))
        ptr.append(ptr[-1] + b.size)
    iv = np.array(starts, dtype=np.int64).reshape(-1, 2)
    return np.array(ptr, dtype=np.int64), iv


def sparse_select(q, k, text: Tuple[int, int], extra: Tuple[int, int], mode: str, param: float,
                  score_scale: Optional[float] = None, topk_override: Optional[int] = None,
                  block: int = BLOCK) -> dict:
    """The whole selection step for q [B, H, Lq, d] and k [B, H, Lk, d]: pool, score, force,
    select, encode. Returns a dict with qbar, kbar, scores (S in Top-K mode, p in mass mode),
    kept [B, H, nQB, nKB], row_ptr and col_idx (rows ordered (b * H + h) * nQB + i)."""
    qbar = pool(q, block)
    kbar = pool(k, block)
    s = block_scores(qbar, kbar, score_scale)
    nkb = s.shape[-1]
    forced = forced_blocks(nkb, text, extra)
    if mode == "topk":
        kk = topk_budget(param, int((~forced).sum())) if topk_override is None else int(topk_override)
        kept = select_topk(s, forced, kk)
        scores = s
    elif mode == "mass":
        scores = block_softmax(s)
        kept = select_mass(scores, forced, param)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    row_ptr, col_idx = to_csr(kept)
    return {"qbar": qbar, "kbar": kbar, "scores": scores, "kept": kept, "row_ptr": row_ptr,
            "col_idx": col_idx, "forced": forced}
