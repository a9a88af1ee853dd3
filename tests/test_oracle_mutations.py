"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and check that the
pins in test_oracle_pins.py catch each of them. A pin set that lets a mutation through is too
weak."""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as oatt
import oracle.energy as oen
import oracle.anchor as oanc
import oracle.select as osel
import oracle.vote as ovote
from tests import test_oracle_pins as pins


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def _scores_unscaled(qbar, kbar, scale=None):
    return np.matmul(np.asarray(qbar, np.float64), np.swapaxes(np.asarray(kbar, np.float64), -1, -2))


def _scores_sqrt_wrong(qbar, kbar, scale=None):
    d = qbar.shape[-1]
    return np.matmul(np.asarray(qbar, np.float64), np.swapaxes(np.asarray(kbar, np.float64), -1, -2)) / d


def _topk_ascending(scores, forced, k):
    return osel._orig_select_topk(-np.asarray(scores, np.float64), forced, k)


def _topk_ties_high(scores, forced, k):
    s = np.asarray(scores, np.float64)
    flipped = s[..., ::-1]
    return osel._orig_select_topk(flipped, forced[::-1], k)[..., ::-1]


def _budget_floor(density, n):
    return min(n, int(math.floor(density * n)))


def _mass_strict(p, forced, tau):
    # "reaches" taken as strictly greater: bump the threshold by one unit
    orig = osel.mass_threshold_units
    try:
        osel.mass_threshold_units = lambda t: orig(t) + 1
        return osel._orig_select_mass(p, forced, tau)
    finally:
        osel.mass_threshold_units = orig


def _mass_ignore_forced(p, forced, tau):
    kept = osel._orig_select_mass(np.where(forced, 0.0, np.asarray(p, np.float64)), forced, tau)
    return kept


def _energy_no_divisor(q, k, rows, scale=None, block=oracle.BLOCK):
    return oen._orig_block_energy_rows(q, k, rows, scale, block) * block


def _energy_transposed(q, k, rows, scale=None, block=oracle.BLOCK):
    # sums over the key axis first and reports per-query-token mass (a transposed reduction)
    e = oen._orig_block_energy_rows(q, k, rows, scale, block)
    return e[:, ::-1].copy()


def _upper_bound_smallest(q, k, rows, budgets, scale=None, block=oracle.BLOCK):
    # the m smallest probabilities instead of the m largest
    rows, budgets = list(rows), list(budgets)
    n_keys = k.shape[-2]
    return 1.0 - oen._orig_token_upper_bound(q, k, rows, [n_keys - m for m in budgets], scale,
                                             block)


def _upper_bound_off_by_one(q, k, rows, budgets, scale=None, block=oracle.BLOCK):
    return oen._orig_token_upper_bound(q, k, rows, [max(m - 1, 0) for m in budgets], scale, block)


def _anchors_from_zero(rows_per_frame, n_anchors):
    # equally spaced starting at row 0 instead of band centres
    return np.array([(j * rows_per_frame) // n_anchors for j in range(n_anchors)], dtype=np.int64)


def _nearest_ties_high(rows_per_frame, n_anchors):
    a = oanc.anchor_rows(rows_per_frame, n_anchors)
    return np.array([max(range(a.size), key=lambda j: (-abs(r - a[j]), j))
                     for r in range(rows_per_frame)], dtype=np.int64)


def _softmax_weighted_unnormalised(logits, values):
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    return e @ values, (m + np.log(e.sum(axis=-1, keepdims=True)))[..., 0]


def _pool_sum(x, block=oracle.BLOCK):
    # block sums instead of block means
    x = np.asarray(x, np.float64)
    return osel._orig_pool(x, block) * np.array(
        [len(osel.block_tokens(i, x.shape[-2], block)) for i in range(osel.n_blocks(x.shape[-2],
                                                                                   block))])[:, None]


def _pool_partial_by_block(x, block=oracle.BLOCK):
    # a partial last block divided by the full block size
    x = np.asarray(x, np.float64)
    out = osel._orig_pool(x, block)
    n_last = len(osel.block_tokens(out.shape[-2] - 1, x.shape[-2], block))
    out[..., -1, :] *= n_last / block
    return out


def _pool_across_heads(x, block=oracle.BLOCK):
    # pooled over the heads as well (a shared mean for every head)
    out = osel._orig_pool(x, block)
    if out.ndim >= 3:
        out = np.broadcast_to(out.mean(axis=-3, keepdims=True), out.shape).copy()
    return out


def _attention_rows_unscaled(q, k, v, row_ptr, col_idx, rows=None, scale=None, block=oracle.BLOCK):
    # the 1/sqrt(d) logit scale left out
    return oatt._orig_attention_rows(q, k, v, row_ptr, col_idx, rows,
                                     1.0 if scale is None else scale, block)


def _topk_without_forced(scores, forced, k):
    # the forced blocks are not added to the kept set
    kept = osel._orig_select_topk(scores, forced, k)
    kept[..., forced] = False
    return kept


def _topk_forced_count_toward_k(scores, forced, k):
    # the forced blocks use up part of the Top-K budget
    return osel._orig_select_topk(scores, forced, max(k - int(np.sum(forced)), 0))


def _mass_candidates_only(p, forced, tau):
    # energies renormalised over the candidate blocks before the prefix is taken
    p = np.asarray(p, np.float64)
    c = np.where(forced, 0.0, p)
    total = c.sum(axis=-1, keepdims=True)
    c = np.divide(c, total, out=np.zeros_like(c), where=total > 0)
    return osel._orig_select_mass(np.where(forced, p, c), forced, tau)


def _csr_descending(kept):
    row_ptr, col_idx = osel._orig_to_csr(kept)
    col_idx = col_idx.copy()
    for r in range(row_ptr.size - 1):
        col_idx[row_ptr[r]:row_ptr[r + 1]] = col_idx[row_ptr[r]:row_ptr[r + 1]][::-1]
    return row_ptr, col_idx


def _csr_inclusive_ptr(kept):
    row_ptr, col_idx = osel._orig_to_csr(kept)
    return np.concatenate([row_ptr[1:], row_ptr[-1:]]), col_idx


def _vote_strict(masks, rho):
    masks = np.asarray(masks, dtype=bool)
    return masks.mean(axis=0) > rho


def _intervals_closed(kept):
    ptr, iv = osel._orig_to_intervals(kept)
    iv = iv.copy()
    iv[:, 1] -= 1
    return ptr, iv


MUTATIONS = {
    "scores without 1/sqrt(d)": (osel, "block_scores", _scores_unscaled,
                                 [pins.test_scores_closed_form_asymmetric, pins.test_mean_field_identity]),
    "scores scaled by 1/d": (osel, "block_scores", _scores_sqrt_wrong,
                             [pins.test_scores_closed_form_asymmetric]),
    "Top-K ascending": (osel, "select_topk", _topk_ascending, [pins.test_topk_golden]),
    "Top-K ties to the higher index": (osel, "select_topk", _topk_ties_high, [pins.test_topk_golden]),
    "budget rounded down": (osel, "topk_budget", _budget_floor, [pins.test_topk_golden]),
    "mass uses strict >": (osel, "select_mass", _mass_strict, [pins.test_mass_golden]),
    "mass ignores forced blocks": (osel, "select_mass", _mass_ignore_forced, [pins.test_mass_golden]),
    "energy without 1/B": (oen, "block_energy_rows", _energy_no_divisor,
                           [pins.test_energy_rows_sum_to_one]),
    "attention without normalisation": (oatt, "_softmax_weighted", _softmax_weighted_unnormalised,
                                        [pins.test_density_one_equals_dense_toy]),
    "energy with reversed key blocks": (oen, "block_energy_rows", _energy_transposed,
                                        [pins.test_energy_equals_sdpa_of_block_indicators,
                                         pins.test_mean_field_identity]),
    "upper bound from the smallest probabilities": (
        oen, "token_upper_bound", _upper_bound_smallest,
        [pins.test_token_upper_bound_brute_force_and_bounds]),
    "anchors start at row 0": (oanc, "anchor_rows", _anchors_from_zero,
                               [pins.test_anchor_rows_are_band_centres]),
    "nearest anchor ties high": (oanc, "nearest_anchor", _nearest_ties_high,
                                 [pins.test_anchor_rows_are_band_centres]),
    "upper bound one token short": (oen, "token_upper_bound", _upper_bound_off_by_one,
                                    [pins.test_token_upper_bound_brute_force_and_bounds,
                                     pins.test_token_upper_bound_mean_field_equals_block_topk]),
    "pool sums instead of averaging": (osel, "pool", _pool_sum, [pins.test_pool_closed_form]),
    "partial block divided by 128": (osel, "pool", _pool_partial_by_block,
                                     [pins.test_pool_partial_block_closed_form]),
    "pool across heads": (osel, "pool", _pool_across_heads, [pins.test_pool_keeps_heads_apart]),
    "attention without 1/sqrt(d)": (oatt, "attention_rows", _attention_rows_unscaled,
                                    [pins.test_partial_blocks_match_sdpa_and_sum_to_one]),
    "Top-K leaves the forced blocks out": (osel, "select_topk", _topk_without_forced,
                                           [pins.test_topk_golden]),
    "forced blocks use up the Top-K budget": (osel, "select_topk", _topk_forced_count_toward_k,
                                              [pins.test_topk_golden]),
    "mass renormalised over candidates": (osel, "select_mass", _mass_candidates_only,
                                          [pins.test_mass_golden,
                                           pins.test_mass_forced_energy_is_not_renormalised]),
    "CSR columns descending": (osel, "to_csr", _csr_descending, [pins.test_csr_closed_form]),
    "CSR row pointers inclusive": (osel, "to_csr", _csr_inclusive_ptr,
                                   [pins.test_csr_closed_form]),
    "vote uses strict >": (ovote, "vote_masks", _vote_strict, [pins.test_vote_worked_example]),
    "intervals closed at the end": (osel, "to_intervals", _intervals_closed,
                                    [pins.test_intervals_hand_example_and_round_trip]),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    module, attr, fn, tests = MUTATIONS[name]
    orig = getattr(module, attr)
    monkeypatch.setattr(module, "_orig_" + attr, orig, raising=False)
    monkeypatch.setattr(module, attr, fn)
    # the package re-exports the names; patch those too so pins that call oracle.X see it
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    caught = [t.__name__ for t in tests if _fails(t)]
    assert caught, f"no pin caught the mutation: {name}"
