"""Comparison helpers shared by the GPU parity tests, the smoke check and the benchmark's
sampled checks. They call only the oracle on host copies of the inputs and results."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

BLOCK = oracle.BLOCK

# Tolerances (stated once, used everywhere)
SCORE_RTOL = 1e-3          # pooled scores: 1e-3 relative ...
SCORE_FLOOR = 1e-2         # ... of max(|S|, 1e-2 * |qbar||kbar| / sqrt(d)) (cancellation floor)
P_RTOL = 1e-3              # mass-mode energies: 1e-3 relative where p >= 1e-6
P_ATOL_SMALL = 1e-9        # ... else absolute
F32_O_MAX = 1e-5           # fp32 inputs: max |O - O_ref|
BF16_O_MAX = 2e-2          # bf16 inputs: max |O - O_ref| ...
BF16_O_MEAN = 2e-3         # ... and mean |O - O_ref|
F32_LSE = 1e-5
# bf16 path: the softmax normaliser is the sum of the bf16-rounded probabilities that weight V
# (round to nearest even, relative error <= 2^-9 each), so lse may differ from the exact value
# by up to ln(1 + 2^-9) = 1.95e-3, plus fp32 rounding
BF16_LSE = 2e-3
# token-level block energy (dense softmax, fp32 accumulation on both input types)
TOK_E_RTOL = 2e-4          # |E - E_ref| <= TOK_E_RTOL * E_ref + TOK_E_ATOL
TOK_E_ATOL = 1e-7
TOK_ROW_SUM = 1e-4         # |sum_c E_rc - 1|
TOK_LSE = 1e-4             # per-query log-sum-exp over all keys (natural log)


def host(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a device tensor (bf16 and fp32 widen exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_scores(s_gpu: np.ndarray, qbar: np.ndarray, kbar: np.ndarray, scale: float):
    """s_gpu [nqb, nkb] for one (b, h) against the oracle's S from its own pooled vectors."""
    s_ref = oracle.block_scores(qbar, kbar, scale)
    bound = np.linalg.norm(qbar, axis=-1)[:, None] * np.linalg.norm(kbar, axis=-1)[None, :] * scale
    tol = SCORE_RTOL * np.maximum(np.abs(s_ref), SCORE_FLOOR * bound)
    err = np.abs(s_gpu - s_ref)
    assert (err <= tol).all(), f"score mismatch: worst excess {float((err - tol).max()):.3e}"
    return float((err / np.maximum(np.abs(s_ref), 1e-30)).max())


def check_energies(p_gpu: np.ndarray, p_ref: np.ndarray):
    big = p_ref >= 1e-6
    rel = np.abs(p_gpu - p_ref) / np.where(big, p_ref, 1.0)
    assert (rel[big] <= P_RTOL).all(), f"energy mismatch: max rel {float(rel[big].max()):.3e}"
    small_err = np.abs(p_gpu - p_ref)[~big]
    assert small_err.size == 0 or small_err.max() <= P_ATOL_SMALL, "small energies off"
    sums = p_gpu.sum(axis=-1)
    assert np.abs(sums - 1.0).max() <= 1e-5


def csr_to_kept(row_ptr: np.ndarray, col_idx: np.ndarray, nkb: int) -> np.ndarray:
    rows = row_ptr.size - 1
    kept = np.zeros((rows, nkb), dtype=bool)
    for r in range(rows):
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        assert (np.diff(cols) > 0).all(), f"row {r}: col_idx not strictly ascending"
        assert cols.size == 0 or (cols[0] >= 0 and cols[-1] < nkb), f"row {r}: index out of range"
        kept[r, cols] = True
    return kept


def csr_to_kept_fast(row_ptr: np.ndarray, col_idx: np.ndarray, nkb: int) -> np.ndarray:
    """Vectorised decode with the same structural checks (for large row counts)."""
    rows = row_ptr.size - 1
    counts = np.diff(row_ptr)
    assert (counts >= 0).all()
    nnz = int(row_ptr[-1])
    cols = col_idx[:nnz].astype(np.int64)
    assert cols.size == 0 or (cols.min() >= 0 and cols.max() < nkb), "index out of range"
    row_of = np.repeat(np.arange(rows), counts)
    if nnz > 1:
        same_row = row_of[1:] == row_of[:-1]
        assert (np.diff(cols)[same_row] > 0).all(), "col_idx not strictly ascending in a row"
    kept = np.zeros((rows, nkb), dtype=bool)
    kept[row_of, cols] = True
    return kept


def check_attention(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray,
                    bf16_inputs: bool):
    err = np.abs(o_gpu - o_ref)
    finite = np.isfinite(lse_ref)
    if bf16_inputs:
        assert err.max() <= BF16_O_MAX, f"O max err {err.max():.3e}"
        assert err.mean() <= BF16_O_MEAN, f"O mean err {err.mean():.3e}"
        ltol = BF16_LSE
    else:
        assert err.max() <= F32_O_MAX, f"O max err {err.max():.3e}"
        ltol = F32_LSE
    if lse_gpu is not None:
        assert (np.isneginf(lse_gpu) == ~finite).all(), "empty-row lse must be -inf"
        if finite.any():
            le = np.abs(lse_gpu[finite] - lse_ref[finite])
            assert le.max() <= ltol, f"lse err {le.max():.3e}"
    return float(err.max()), float(err.mean())


def topk_near_tie_ok(kept_gpu, kept_ref, s_ref, forced, tol):
    """Where the GPU mask (selected on GPU scores) differs from the oracle's own mask, every
    swapped block must sit within `tol` of the oracle's selection threshold."""
    diff_rows = np.flatnonzero((kept_gpu != kept_ref).any(axis=1))
    for r in diff_rows:
        only_gpu = kept_gpu[r] & ~kept_ref[r]
        only_ref = kept_ref[r] & ~kept_gpu[r]
        lo = s_ref[r][kept_ref[r] & ~forced].min()
        assert (np.abs(s_ref[r][only_gpu] - lo) <= 2 * tol[r][only_gpu]).all()
        assert (np.abs(s_ref[r][only_ref] - lo) <= 2 * tol[r][only_ref]).all()
    return diff_rows.size


def check_token_energy(e_gpu: np.ndarray, e_ref: np.ndarray):
    """Token-level energies against the oracle's Eq. (5) on the same rows."""
    err = np.abs(e_gpu - e_ref)
    tol = TOK_E_RTOL * e_ref + TOK_E_ATOL
    assert (err <= tol).all(), f"energy mismatch: worst excess {float((err - tol).max()):.3e}"
    assert np.abs(e_gpu.sum(axis=-1) - 1.0).max() <= TOK_ROW_SUM
    assert (e_gpu >= 0).all()


def rows_to_tokens(o_rows: np.ndarray, lse_rows: np.ndarray, batch: int, heads: int, lq: int):
    """Oracle attention per CSR row ([rows, 128, d], [rows, 128]) -> per token ([B, H, lq, d],
    [B, H, lq]), dropping the slots past the end of a partial last query block."""
    nqb = -(-lq // BLOCK)
    d = o_rows.shape[-1]
    o = o_rows.reshape(batch, heads, nqb * BLOCK, d)[:, :, :lq]
    lse = lse_rows.reshape(batch, heads, nqb * BLOCK)[:, :, :lq]
    return o, lse
