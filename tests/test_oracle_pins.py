"""Pins of the oracle against facts fixed outside it: hand-worked examples, closed forms,
invariants of the definitions, brute force on tiny inputs and independent library routines.

Each test names what a plausible mistake in the oracle would break.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from synth import BLOCK, WORKLOADS, make_qkv, small_variants

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- partition and pooling

def test_partition_counts():
    assert oracle.n_blocks(1024) == 8
    assert oracle.n_blocks(144896) == 1132
    # a partial last block holds the remaining tokens (the DiT's 75,600 video tokens: 590 full
    # blocks and one of 80)
    assert oracle.n_blocks(75600) == 591 and oracle.n_blocks(127) == 1 and oracle.n_blocks(129) == 2
    assert list(oracle.select.block_tokens(590, 75600)) == list(range(75520, 75600))
    for bad in (0, -128):
        with pytest.raises(ValueError):
            oracle.n_blocks(bad)


def test_pool_partial_block_closed_form():
    # x[t] = t: a full block averages to 128 i + 63.5; the partial last block of L = 300 tokens
    # (tokens 256 .. 299) averages to 277.5
    L = 300
    x = np.arange(L, dtype=np.float64)[:, None] * np.ones((1, 2))
    np.testing.assert_array_equal(oracle.pool(x)[:, 0], [63.5, 191.5, 277.5])


def test_partial_blocks_match_sdpa_and_sum_to_one():
    # lengths that are not block multiples: the masked and gathered attention agree with torch's
    # float64 SDPA over the valid tokens, and token-level energies still sum to 1 per row
    rng = np.random.default_rng(41)
    lq, lk, d = 2 * BLOCK + 37, 3 * BLOCK + 5, 8
    q = rng.standard_normal((1, 2, lq, d))
    k = rng.standard_normal((1, 2, lk, d))
    v = rng.standard_normal((1, 2, lk, d))
    nqb, nkb = oracle.n_blocks(lq), oracle.n_blocks(lk)
    kept = rng.random((1, 2, nqb, nkb)) < 0.6
    kept[..., nkb - 1] = True                       # the partial key block is always used
    row_ptr, col_idx = oracle.to_csr(kept.reshape(-1, nkb))
    o1, l1 = oracle.attention_rows(q, k, v, row_ptr, col_idx)
    o1 = o1.reshape(1, 2, nqb * BLOCK, d)[:, :, :lq]
    l1 = l1.reshape(1, 2, nqb * BLOCK)[:, :, :lq]
    o2, l2 = oracle.attention_masked(q, k, v, kept)
    mask = torch.from_numpy(np.repeat(np.repeat(kept, BLOCK, axis=-2), BLOCK, axis=-1)[..., :lq, :lk])
    o3 = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask).numpy()
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o1, o3, rtol=1e-10, atol=1e-12)
    e = oracle.block_energy_rows(q, k, rows=range(2 * nqb))
    np.testing.assert_allclose(e.sum(axis=1), 1.0, atol=1e-12)
    # energies against SDPA over block indicators, with the partial query block's own count
    ind = np.zeros((lk, nkb))
    ind[np.arange(lk), np.arange(lk) // BLOCK] = 1.0
    o_ind = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k),
        torch.from_numpy(np.broadcast_to(ind, (1, 2, lk, nkb)).copy())).numpy()
    for r in range(2 * nqb):
        h, i = divmod(r, nqb)
        t0, t1 = i * BLOCK, min((i + 1) * BLOCK, lq)
        np.testing.assert_allclose(e[r], o_ind[0, h, t0:t1].mean(axis=0), rtol=1e-12, atol=1e-15)


def test_pool_closed_form():
    # x[t, j] = t + 1000 j: the mean over block i is 128 i + 63.5 + 1000 j.
    # Pins the block size, the pooled axis and the divisor.
    L, d = 4 * BLOCK, 3
    t = np.arange(L, dtype=np.float64)[:, None]
    j = np.arange(d, dtype=np.float64)[None, :]
    x = (t + 1000.0 * j)[None, None]
    got = oracle.pool(x)
    want = (128.0 * np.arange(4)[:, None] + 63.5 + 1000.0 * j)[None, None]
    np.testing.assert_array_equal(got, want)


def test_pool_keeps_heads_apart():
    x = np.zeros((1, 2, BLOCK, 2))
    x[0, 0] = 1.0
    x[0, 1] = -3.0
    got = oracle.pool(x)
    np.testing.assert_array_equal(got[0, 0, 0], [1.0, 1.0])
    np.testing.assert_array_equal(got[0, 1, 0], [-3.0, -3.0])


# ---------------------------------------------------------------- block scores

def test_scores_closed_form_asymmetric():
    # Query block i holds (i+1) e_i in every token; key block c holds a_c with a_c[j] = (c+1)(j+1).
    # Then S_ic = (i+1) * a_c[i] / sqrt(d) = (i+1)^2 (c+1) / sqrt(d): not symmetric in (i, c),
    # so a transposed product or a missing / wrong scale fails.
    d, nqb, nkb = 4, 3, 5
    q = np.zeros((1, 1, nqb * BLOCK, d))
    for i in range(nqb):
        q[0, 0, i * BLOCK:(i + 1) * BLOCK, i] = i + 1
    k = np.zeros((1, 1, nkb * BLOCK, d))
    for c in range(nkb):
        k[0, 0, c * BLOCK:(c + 1) * BLOCK, :] = (c + 1) * (np.arange(d) + 1)
    s = oracle.block_scores(oracle.pool(q), oracle.pool(k))[0, 0]
    want = np.array([[(i + 1) ** 2 * (c + 1) / math.sqrt(d) for c in range(nkb)] for i in range(nqb)])
    np.testing.assert_allclose(s, want, rtol=1e-15, atol=0)


def test_scores_equal_mean_token_logit():
    # Bilinearity: the score of two pooled blocks is the mean of the 128 x 128 token logits
    # q_t . k_s / sqrt(d). Computed here by brute force over token pairs.
    rng = np.random.default_rng(1)
    d = 8
    q = rng.standard_normal((1, 1, 2 * BLOCK, d))
    k = rng.standard_normal((1, 1, 3 * BLOCK, d))
    s = oracle.block_scores(oracle.pool(q), oracle.pool(k))[0, 0]
    for i in range(2):
        for c in range(3):
            qi = q[0, 0, i * BLOCK:(i + 1) * BLOCK]
            kc = k[0, 0, c * BLOCK:(c + 1) * BLOCK]
            total = 0.0
            for a in range(BLOCK):
                total += float(np.sum(kc @ qi[a]))
            assert s[i, c] == pytest.approx(total / (BLOCK * BLOCK) / math.sqrt(d), rel=1e-12, abs=1e-13)


# ---------------------------------------------------------------- forced set

def test_forced_ranges():
    m = oracle.forced_blocks(10, (0, 2), (4, 7))
    assert np.flatnonzero(m).tolist() == [0, 1, 4, 5, 6]
    assert not oracle.forced_blocks(5, (0, 0), (0, 0)).any()
    with pytest.raises(ValueError):
        oracle.forced_blocks(5, (0, 3), (2, 4))      # overlap
    with pytest.raises(ValueError):
        oracle.forced_blocks(5, (0, 6), (0, 0))      # outside
    with pytest.raises(ValueError):
        oracle.forced_blocks(5, (3, 2), (0, 0))      # reversed


# ---------------------------------------------------------------- Top-K

def test_topk_golden():
    g = _load("topk_rows.json")
    for case in g["cases"]:
        s = np.array(case["scores"])
        forced = oracle.forced_blocks(s.size, tuple(case["text"]), tuple(case["extra"]))
        k = oracle.topk_budget(case["density"], int((~forced).sum()))
        assert k == case["k"], case["name"]
        kept = oracle.select_topk(s[None], forced, k)[0]
        assert np.flatnonzero(kept).tolist() == case["kept"], case["name"]
    for b in g["budgets"]:
        assert oracle.topk_budget(b["density"], b["candidates"]) == b["k"], b["note"]


def _brute_topk(row, forced, k):
    cand = [c for c in range(len(row)) if not forced[c]]
    # Python compares -0.0 == 0.0, so signed zeros tie and fall back to the index
    order = sorted(cand, key=lambda c: (-row[c], c))
    return sorted(set(np.flatnonzero(forced).tolist()) | set(order[:k]))


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    nkb = int(rng.integers(2, 40))
    rows = rng.integers(-3, 4, size=(25, nkb)).astype(np.float64)   # many ties
    rows[rng.random(rows.shape) < 0.1] = -0.0
    t0 = int(rng.integers(0, nkb))
    forced = oracle.forced_blocks(nkb, (0, t0 // 2), (t0 // 2, t0 // 2 + (t0 % 3 > 0)))
    ncand = int((~forced).sum())
    for k in sorted({0, 1, ncand // 2, ncand}):
        kept = oracle.select_topk(rows, forced, k)
        for r in range(rows.shape[0]):
            assert np.flatnonzero(kept[r]).tolist() == _brute_topk(rows[r].tolist(), forced, k)


def test_topk_all_equal_row_keeps_lowest_indices():
    forced = oracle.forced_blocks(9, (0, 2), (0, 0))
    kept = oracle.select_topk(np.full((1, 9), 0.25), forced, 3)[0]
    assert np.flatnonzero(kept).tolist() == [0, 1, 2, 3, 4]


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10_000), st.floats(0.01, 100.0), st.floats(-50.0, 50.0))
def test_topk_invariant_to_scale_and_shift(seed, a, b):
    # Positive scaling and a per-row shift do not change the order, hence not the mask.
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((4, 23))
    forced = oracle.forced_blocks(23, (0, 3), (0, 0))
    base = oracle.select_topk(s, forced, 6)
    # only compare when the transformed scores keep distinct values distinct in float64
    t = s * a + b
    if len(np.unique(t)) == len(np.unique(s)):
        np.testing.assert_array_equal(oracle.select_topk(t, forced, 6), base)


def test_topk_is_an_order_statistic():
    # Every kept candidate scores at least as high as every dropped candidate.
    rng = np.random.default_rng(7)
    s = rng.standard_normal((50, 31))
    forced = oracle.forced_blocks(31, (0, 4), (10, 12))
    kept = oracle.select_topk(s, forced, 9)
    for r in range(50):
        kc = s[r][kept[r] & ~forced]
        dc = s[r][~kept[r] & ~forced]
        assert kc.size == 9 and kc.min() >= dc.max()


# ---------------------------------------------------------------- mass threshold

def test_mass_golden():
    g = _load("mass_rows.json")
    for case in g["cases"]:
        p = np.array(case["p"])
        forced = np.zeros(p.size, bool)
        forced[case["forced"]] = True
        kept = oracle.select_mass(p[None], forced, case["tau"])[0]
        assert np.flatnonzero(kept).tolist() == case["kept"], case["name"]


def test_mass_forced_energy_is_not_renormalised():
    # The energies are the row's softmax over all key blocks; forced blocks keep theirs and the
    # candidates are not rescaled to the non-forced share. p = (0.5, 0.2, 0.2, 0.1) with block 0
    # forced and tau = 0.8: 0.5 + 0.2 = 0.7 < 0.8, so two candidates are needed (0.9). Rescaling
    # the candidates by 1 / 0.5 would give 0.5 + 0.4 = 0.9 with one.
    p = np.array([[0.5, 0.2, 0.2, 0.1]])
    forced = np.array([True, False, False, False])
    kept = oracle.select_mass(p, forced, 0.8)[0]
    assert np.flatnonzero(kept).tolist() == [0, 1, 2]


def test_mass_units_exact():
    assert int(oracle.mass_units(np.array([0.5]))[0]) == 2 ** 61
    assert int(oracle.mass_units(np.array([2.0 ** -62]))[0]) == 1
    assert int(oracle.mass_units(np.array([2.0 ** -63]))[0]) == 0
    assert oracle.mass_threshold_units(0.75) == 3 * 2 ** 60
    assert oracle.mass_threshold_units(0.9) == math.ceil(0.9 * 2.0 ** 62)


@pytest.mark.parametrize("seed", range(8))
def test_mass_is_minimal_prefix_by_enumeration(seed):
    # Brute force over every subset containing the forced blocks: the kept set has the minimum
    # size among sets whose fixed-point mass reaches the threshold, and it is a prefix of the
    # (energy desc, index asc) order. Catches a wrong sort direction, a strict '>' and
    # forgetting the forced mass.
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(3, 11))
    p = rng.dirichlet(np.full(n, 0.4))
    p[rng.random(n) < 0.2] = p[0]                          # some exact ties
    p = p / p.sum()
    forced = np.zeros(n, bool)
    if seed % 2:
        forced[: int(rng.integers(1, 3))] = True
    tau = float(rng.uniform(0.3, 0.95))
    kept = oracle.select_mass(p[None], forced, tau)[0]
    u = [int(x) for x in oracle.mass_units(p)]
    theta = oracle.mass_threshold_units(tau)
    cand = [c for c in range(n) if not forced[c]]
    fset = [c for c in range(n) if forced[c]]
    best = None
    for size in range(0, len(cand) + 1):
        for sub in itertools.combinations(cand, size):
            if sum(u[c] for c in fset) + sum(u[c] for c in sub) >= theta:
                best = size
                break
        if best is not None:
            break
    if best is None:
        assert kept.all()
        return
    assert int(kept.sum()) - len(fset) == best
    order = sorted(cand, key=lambda c: (-p[c], c))
    assert sorted(np.flatnonzero(kept & ~forced).tolist()) == sorted(order[:best])


def test_mass_shift_invariant():
    # Softmax is invariant to a per-row shift of the scores, so the mass mask is too.
    rng = np.random.default_rng(3)
    s = rng.standard_normal((6, 17)) * 3
    forced = np.zeros(17, bool)
    a = oracle.select_mass(oracle.block_softmax(s), forced, 0.9)
    b = oracle.select_mass(oracle.block_softmax(s + 11.0), forced, 0.9)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- block energy, Eq. (5)

def test_energy_rows_sum_to_one():
    w = small_variants()["star_mid_small"]
    q, k, _ = (t.double().numpy() for t in make_qkv(w.with_(heads=1), seed=5))
    e = oracle.block_energy_rows(q, k, rows=range(w.n_q_blocks))
    np.testing.assert_allclose(e.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert (e >= 0).all()


def test_mean_field_identity():
    # With every token of a block equal to the block's vector, P_ij = exp(S_rc) / (B sum_c'
    # exp(S_rc')) inside block pair (r, c), so Eq. (5) gives E_rc = softmax_c(S_rc) exactly:
    # the pooled-score softmax with scale 1/sqrt(d) is the token-level energy. The two mass
    # masks then agree. Pins the score scale and the energy normalisation together.
    rng = np.random.default_rng(11)
    d, nqb, nkb = 16, 3, 9
    qc = rng.standard_normal((nqb, d)) * 1.5
    kc = rng.standard_normal((nkb, d)) * 1.5
    q = np.repeat(qc, BLOCK, axis=0)[None, None]
    k = np.repeat(kc, BLOCK, axis=0)[None, None]
    e_tok = oracle.block_energy_rows(q, k, rows=range(nqb))
    p = oracle.block_softmax(oracle.block_scores(oracle.pool(q), oracle.pool(k)))[0, 0]
    np.testing.assert_allclose(p, e_tok, rtol=1e-12, atol=1e-15)
    forced = np.zeros(nkb, bool)
    for tau in (0.5, 0.8, 0.95):
        np.testing.assert_array_equal(oracle.select_mass(p, forced, tau),
                                      oracle.select_mass(e_tok, forced, tau))


def test_energy_equals_sdpa_of_block_indicators():
    # With V the one-hot indicator of each key's block, attention output O[t, c] is the
    # probability mass query t puts on block c; Eq. (5) is then the mean of O over the queries
    # of the block. torch's float64 SDPA computes O independently of the oracle's code.
    rng = np.random.default_rng(21)
    bsz, heads, nqb, nkb, d = 1, 2, 2, 5, 16
    q = rng.standard_normal((bsz, heads, nqb * BLOCK, d)) * 2.0
    k = rng.standard_normal((bsz, heads, nkb * BLOCK, d)) * 2.0
    ind = np.repeat(np.eye(nkb), BLOCK, axis=0)                      # [Lk, nKB]
    v = np.broadcast_to(ind, (bsz, heads, nkb * BLOCK, nkb)).copy()
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    want = o.reshape(bsz * heads, nqb, BLOCK, nkb).mean(axis=2).reshape(-1, nkb)
    got = oracle.block_energy_rows(q, k, rows=range(bsz * heads * nqb))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15)


def test_token_upper_bound_brute_force_and_bounds():
    rng = np.random.default_rng(23)
    # tiny blocks: brute force over every key subset of the budget's size
    import itertools
    blk, nqb, nkb, d = 2, 2, 4, 3
    q = rng.standard_normal((1, 1, nqb * blk, d))
    k = rng.standard_normal((1, 1, nkb * blk, d))
    logits = (q[0, 0] @ k[0, 0].T) / math.sqrt(d)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    for m in range(1, nkb * blk + 1):
        best = [max(p[t, list(c)].sum() for c in itertools.combinations(range(nkb * blk), m))
                for t in range(nqb * blk)]
        want = [np.mean(best[r * blk:(r + 1) * blk]) for r in range(nqb)]
        got = oracle.token_upper_bound(q, k, rows=range(nqb), budgets=[m] * nqb, block=blk)
        np.testing.assert_allclose(got, want, rtol=1e-12)
    # full budget keeps everything; any block mask of the same size retains at most the bound
    w = small_variants()["star_mid_small"]
    qq, kk, _ = (t.double().numpy() for t in make_qkv(w.with_(heads=1), seed=6))
    rows = range(w.n_q_blocks)
    np.testing.assert_allclose(
        oracle.token_upper_bound(qq, kk, rows, [w.lk] * w.n_q_blocks), 1.0, atol=1e-12)
    e = oracle.block_energy_rows(qq, kk, rows)
    for nkeep in (1, 3, 7):
        kept = np.zeros_like(e, dtype=bool)
        for r in range(e.shape[0]):
            kept[r, rng.choice(e.shape[1], nkeep, replace=False)] = True
        ub = oracle.token_upper_bound(qq, kk, rows, [nkeep * BLOCK] * e.shape[0])
        assert (oracle.retained_mass(e, kept) <= ub + 1e-12).all()


def test_token_upper_bound_mean_field_equals_block_topk():
    # With every token equal to its block's vector, all queries of a block have the same
    # probabilities, constant within a key block, so their best m = K * 128 tokens are the K
    # blocks of largest energy and the bound equals the retained mass of the block Top-K mask.
    rng = np.random.default_rng(29)
    d, nqb, nkb, kk = 16, 2, 7, 3
    q = np.repeat(rng.standard_normal((nqb, d)), BLOCK, axis=0)[None, None]
    k = np.repeat(rng.standard_normal((nkb, d)) * 1.5, BLOCK, axis=0)[None, None]
    e = oracle.block_energy_rows(q, k, rows=range(nqb))
    kept = np.zeros_like(e, dtype=bool)
    for r in range(nqb):
        kept[r, np.argsort(-e[r], kind="stable")[:kk]] = True
    ub = oracle.token_upper_bound(q, k, range(nqb), [kk * BLOCK] * nqb)
    np.testing.assert_allclose(ub, oracle.retained_mass(e, kept), rtol=1e-12)


# ---------------------------------------------------------------- attention

def _torch_sdpa(q, k, v, kept):
    tq, tk, tv = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (q, k, v))
    if kept is None:
        return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).numpy()
    mask = torch.from_numpy(np.repeat(np.repeat(kept, BLOCK, axis=-2), BLOCK, axis=-1))
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask).numpy()


@pytest.mark.parametrize("seed", range(3))
def test_attention_three_ways(seed):
    # The gather formulation, the -inf masked formulation and torch's SDPA (float64, boolean
    # mask) agree on random masks.
    rng = np.random.default_rng(seed)
    bsz, h, nqb, nkb, d = 1, 2, 2, 4, 8
    q = rng.standard_normal((bsz, h, nqb * BLOCK, d))
    k = rng.standard_normal((bsz, h, nkb * BLOCK, d))
    v = rng.standard_normal((bsz, h, nkb * BLOCK, d))
    kept = rng.random((bsz, h, nqb, nkb)) < 0.5
    kept[..., 0] = True                                  # no empty row for SDPA
    row_ptr, col_idx = oracle.to_csr(kept.reshape(-1, nkb))
    o1, l1 = oracle.attention_rows(q, k, v, row_ptr, col_idx)
    o2, l2 = oracle.attention_masked(q, k, v, kept)
    o3 = _torch_sdpa(q, k, v, kept)
    o1 = o1.reshape(bsz, h, nqb * BLOCK, d)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o1, o3, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l1.reshape(bsz, h, -1), l2, rtol=1e-12, atol=1e-12)
    # lse against a direct log-sum-exp over the kept keys of one query
    qi = q[0, 1, 5]
    cols = np.flatnonzero(kept[0, 1, 0])
    keys = np.concatenate([k[0, 1, c * BLOCK:(c + 1) * BLOCK] for c in cols])
    direct = math.log(sum(math.exp(float(x)) for x in keys @ qi / math.sqrt(d)))
    assert l1.reshape(bsz, h, -1)[0, 1, 5] == pytest.approx(direct, rel=1e-12)


def test_empty_row_gives_zero_output():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, BLOCK, 4))
    k = rng.standard_normal((1, 1, 2 * BLOCK, 4))
    kept = np.zeros((1, 1, 1, 2), bool)
    row_ptr, col_idx = oracle.to_csr(kept.reshape(-1, 2))
    o, lse = oracle.attention_rows(q, k, k, row_ptr, col_idx)
    assert (o == 0).all() and np.isneginf(lse).all()
    o2, lse2 = oracle.attention_masked(q, k, k, kept)
    assert (o2 == 0).all() and np.isneginf(lse2).all()


def test_attention_closed_form_identical_keys():
    # All kept keys identical: uniform weights, O = mean of the kept values, and
    # lse = log(#kept tokens) + q . k / sqrt(d).
    rng = np.random.default_rng(4)
    d = 6
    q = rng.standard_normal((1, 1, BLOCK, d))
    kvec = rng.standard_normal(d)
    k = np.tile(kvec, (1, 1, 3 * BLOCK, 1))
    v = rng.standard_normal((1, 1, 3 * BLOCK, d))
    kept = np.array([True, False, True])
    row_ptr, col_idx = oracle.to_csr(kept[None])
    o, lse = oracle.attention_rows(q, k, v, row_ptr, col_idx)
    vmean = np.concatenate([v[0, 0, :BLOCK], v[0, 0, 2 * BLOCK:]]).mean(axis=0)
    np.testing.assert_allclose(o[0], np.tile(vmean, (BLOCK, 1)), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0], math.log(2 * BLOCK) + q[0, 0] @ kvec / math.sqrt(d),
                               rtol=1e-12)


def test_density_one_equals_dense_toy():
    # Toy workload at density 1.0: every block is kept and the sparse result equals dense
    # attention (the oracle's own dense path and torch SDPA).
    w = WORKLOADS["toy_dense"]
    q, k, v = (t.double().numpy() for t in make_qkv(w, seed=0))
    sel = oracle.sparse_select(q, k, w.text, w.extra, w.mode, w.param)
    assert sel["kept"].all()
    o, lse = oracle.attention_rows(q, k, v, sel["row_ptr"], sel["col_idx"])
    od, lsed = oracle.attention_dense(q, k, v)
    np.testing.assert_allclose(o.reshape(od.shape), od, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o.reshape(od.shape), _torch_sdpa(q, k, v, None), rtol=1e-10, atol=1e-12)


def test_within_block_permutation():
    # Permuting tokens inside blocks leaves pooled vectors and masks unchanged, and permutes
    # the output rows the same way.
    w = small_variants()["star_mid_small"].with_(heads=1)
    q, k, v = (t.double().numpy() for t in make_qkv(w, seed=2))
    rng = np.random.default_rng(0)
    pq = np.concatenate([b * BLOCK + rng.permutation(BLOCK) for b in range(w.n_q_blocks)])
    pk = np.concatenate([b * BLOCK + rng.permutation(BLOCK) for b in range(w.n_k_blocks)])
    a = oracle.sparse_select(q, k, w.text, w.extra, "topk", w.param)
    b = oracle.sparse_select(q[:, :, pq], k[:, :, pk], w.text, w.extra, "topk", w.param)
    np.testing.assert_allclose(a["qbar"], b["qbar"], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(a["kept"], b["kept"])
    oa, _ = oracle.attention_rows(q, k, v, a["row_ptr"], a["col_idx"])
    ob, _ = oracle.attention_rows(q[:, :, pq], k[:, :, pk], v[:, :, pk], b["row_ptr"], b["col_idx"])
    np.testing.assert_allclose(oa.reshape(-1, w.head_dim)[pq], ob.reshape(-1, w.head_dim), rtol=1e-10,
                               atol=1e-12)


# ---------------------------------------------------------------- CSR and the whole selection

@pytest.mark.parametrize("name", list(small_variants()))
def test_select_structure_small_workloads(name):
    w = small_variants()[name]
    q, k, _ = (t.double().numpy() for t in make_qkv(w, seed=1))
    sel = oracle.sparse_select(q, k, w.text, w.extra, w.mode, w.param)
    rp, ci = sel["row_ptr"], sel["col_idx"]
    forced = np.flatnonzero(sel["forced"])
    ncand = w.n_k_blocks - forced.size
    assert rp[0] == 0 and rp.size == w.rows + 1 and ci.size == rp[-1]
    for r in range(w.rows):
        cols = ci[rp[r]:rp[r + 1]]
        assert (np.diff(cols) > 0).all()
        assert set(forced.tolist()) <= set(cols.tolist())
        if w.mode == "topk":
            assert cols.size == forced.size + oracle.topk_budget(w.param, ncand)
    if w.mode == "mass":
        p = sel["scores"].reshape(-1, w.n_k_blocks)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
        kept = sel["kept"].reshape(-1, w.n_k_blocks)
        assert (np.where(kept, p, 0).sum(axis=1) >= w.param - 1e-12).all()


def test_csr_closed_form():
    kept = np.array([[1, 0, 1], [0, 0, 0], [1, 1, 1]], bool)
    rp, ci = oracle.to_csr(kept)
    assert rp.tolist() == [0, 2, 2, 5]
    assert ci.tolist() == [0, 2, 0, 1, 2]


# ---------------------------------------------------------------- cross-input vote

def test_vote_worked_example():
    g = _load("vote_example.json")
    n = g["n_inputs"]
    counts = g["counts"]
    masks = np.zeros((n, len(counts)), bool)
    for j, c in enumerate(counts):
        masks[:c, j] = True
    assert oracle.vote_masks(masks, g["rho"]).tolist() == g["kept"]


# ---------------------------------------------------------------- anchor rows (repeating heads)

def test_anchor_rows_are_band_centres():
    # the page's default of 5 anchors on the 45 rows of a Wan 720p latent frame
    assert oracle.anchor_rows(45, 5).tolist() == [4, 13, 22, 31, 40]
    assert oracle.anchor_rows(7, 7).tolist() == list(range(7))
    assert oracle.anchor_rows(10, 1).tolist() == [5]
    near = oracle.nearest_anchor(45, 5)
    # bands of 9 rows map to their centre; every row is at most 4 rows from its anchor
    assert near.tolist() == [r // 9 for r in range(45)]
    assert oracle.anchor_rows(6, 2).tolist() == [1, 4]
    assert oracle.nearest_anchor(6, 2).tolist() == [0, 0, 0, 1, 1, 1]
    # ties go to the lower anchor: anchors at rows 2 and 6 of 8, row 4 is 2 away from both
    assert oracle.anchor_rows(8, 2).tolist() == [2, 6]
    assert oracle.nearest_anchor(8, 2).tolist() == [0, 0, 0, 0, 0, 1, 1, 1]


def _dense(q, k, v):
    return oracle.attention_dense(q, k, v)


def test_anchor_path_reduces_to_dense():
    rng = np.random.default_rng(31)
    b, h, frames, rows, width, d = 1, 2, 2, 4, 16, 8
    lq = frames * rows * width + 20                      # a trailing partial block
    q = rng.standard_normal((b, h, lq, d))
    k = rng.standard_normal((b, h, 96, d))
    v = rng.standard_normal((b, h, 96, d))
    o_d, l_d = _dense(q, k, v)
    # every row its own anchor: exactly dense attention
    o, l = oracle.anchor_attention(q, k, v, frames, rows, width, rows)
    np.testing.assert_allclose(o, o_d, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, l_d, rtol=1e-12, atol=1e-12)
    # fewer anchors: anchor rows and the tail are dense; other rows copy their anchor's row
    o, l = oracle.anchor_attention(q, k, v, frames, rows, width, 2)
    a = oracle.anchor_rows(rows, 2)
    near = oracle.nearest_anchor(rows, 2)
    for f in range(frames):
        for r in range(rows):
            t = f * rows * width + r * width
            src = f * rows * width + a[near[r]] * width
            np.testing.assert_allclose(o[:, :, t:t + width], o_d[:, :, src:src + width],
                                       rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o[:, :, frames * rows * width:], o_d[:, :, frames * rows * width:],
                               rtol=1e-12, atol=1e-12)


def test_anchor_path_exact_on_repeating_rows():
    # a perfectly repeating head: every spatial row of a frame has the same queries, so the
    # broadcast loses nothing and the anchor path equals dense attention
    rng = np.random.default_rng(37)
    frames, rows, width, d = 3, 6, 8, 16
    row_q = rng.standard_normal((frames, 1, width, d))
    q = np.broadcast_to(row_q, (frames, rows, width, d)).reshape(1, 1, -1, d).copy()
    k = rng.standard_normal((1, 1, 64, d))
    v = rng.standard_normal((1, 1, 64, d))
    o, l = oracle.anchor_attention(q, k, v, frames, rows, width, 2)
    o_d, l_d = _dense(q, k, v)
    np.testing.assert_allclose(o, o_d, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, l_d, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- interval skip list

def test_intervals_hand_example_and_round_trip():
    kept = np.array([[1, 1, 0, 1, 0, 0, 1, 1],
                     [0, 0, 0, 0, 0, 0, 0, 0],
                     [1, 1, 1, 1, 1, 1, 1, 1],
                     [0, 1, 0, 1, 0, 1, 0, 1]], dtype=bool)
    ptr, iv = oracle.to_intervals(kept)
    assert ptr.tolist() == [0, 3, 3, 4, 8]
    assert iv.tolist() == [[0, 2], [3, 4], [6, 8], [0, 8], [1, 2], [3, 4], [5, 6], [7, 8]]
    rng = np.random.default_rng(43)
    for density in (0.05, 0.5, 0.95):
        kept = rng.random((9, 77)) < density
        ptr, iv = oracle.to_intervals(kept)
        back = np.zeros_like(kept)
        for r in range(kept.shape[0]):
            for s_, e_ in iv[ptr[r]:ptr[r + 1]]:
                assert s_ < e_
                back[r, s_:e_] = True
            runs = iv[ptr[r]:ptr[r + 1]]
            assert (runs[1:, 0] > runs[:-1, 1]).all()      # maximal: runs never touch
        np.testing.assert_array_equal(back, kept)
