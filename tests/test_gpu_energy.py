"""GPU parity of the token-level block energy (CalibAtt Eq. (5)), the retained mass of a mask and
the cumulative-mass selection on token-level energies, through the C ABI, against the oracle.

Bars: energies within 2e-4 relative + 1e-7 absolute of the float64 oracle on the same (bf16 or
fp32) input values, every row summing to 1 within 1e-4; the per-query lse within 1e-4; masks
bit-exact against the oracle selecting from the GPU's own energies; retained mass equal to the
oracle's float64 sum of the GPU's energies over the GPU's mask (1e-12 relative).
"""
import numpy as np
import pytest
import torch

import oracle
from synth import BLOCK, WORKLOADS, make_qkv, small_variants
from tests import parity as P

pytestmark = pytest.mark.gpu


def dbsp():
    import dynamic_block_sparse_pool_amd as m
    return m


def say(msg):
    print(f"[gpu-energy] {msg}", flush=True)


def forced_of(w):
    return oracle.forced_blocks(w.n_k_blocks, w.text, w.extra)


@pytest.mark.parametrize("name", ["toy", "star_mid_small", "clip1_small", "final_small",
                                  "dit_mass_small"])
def test_energy_parity(name):
    w = small_variants()[name]
    say(f"case {name} B={w.batch} H={w.heads} Lq={w.lq} Lk={w.lk} d={w.head_dim} {w.dtype}")
    q, k, _ = make_qkv(w, device="cuda", seed=4)
    e, lse = dbsp().block_energy(q, k, return_lse=True)
    torch.cuda.synchronize()
    qh, kh = P.host(q), P.host(k)
    e_ref = oracle.block_energy_rows(qh, kh, rows=range(w.rows))
    P.check_token_energy(P.host(e), e_ref)
    _, lse_ref = oracle.attention_dense(qh, kh, kh)
    assert np.abs(P.host(lse) - lse_ref).max() <= P.TOK_LSE


def test_energy_edge_shapes():
    m = dbsp()
    # one key block: every energy is 1; one query block against many key blocks
    for lq, lk in ((128, 128), (128, 37 * 128), (5 * 128, 128)):
        w = small_variants()["star_mid_small"].with_(heads=2, lq=lq, lk=lk)
        say(f"case edge lq={lq} lk={lk}")
        q, k, _ = make_qkv(w, device="cuda", seed=9)
        e = P.host(m.block_energy(q, k))
        torch.cuda.synchronize()
        e_ref = oracle.block_energy_rows(P.host(q), P.host(k), rows=range(w.rows))
        P.check_token_energy(e, e_ref)
        if lk == 128:
            np.testing.assert_allclose(e, 1.0, rtol=0, atol=P.TOK_ROW_SUM)


def test_energy_deterministic():
    w = small_variants()["final_small"]
    say("case determinism final_small")
    q, k, _ = make_qkv(w, device="cuda", seed=2)
    a = dbsp().block_energy(q, k)
    b = dbsp().block_energy(q, k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["dit_mass_small", "clip1_small", "toy"])
def test_select_energy_and_retained_mass(name):
    m = dbsp()
    w = small_variants()[name]
    say(f"case select_energy {name}")
    q, k, _ = make_qkv(w, device="cuda", seed=5)
    e = m.block_energy(q, k)
    torch.cuda.synchronize()
    eh = P.host(e)
    nkb = w.n_k_blocks
    forced = forced_of(w)
    for tau in (0.3, 0.9, 0.999, 1.0):
        idx = m.select_energy(e, tau, w.text, w.extra, batch=w.batch, heads=w.heads)
        mass = m.retained_mass(e, idx, batch=w.batch, heads=w.heads)
        torch.cuda.synchronize()
        rp = idx.row_ptr.cpu().numpy().astype(np.int64)
        ci = idx.col_idx.cpu().numpy().astype(np.int64)
        kept_gpu = P.csr_to_kept(rp, ci, nkb)
        kept_ora = oracle.select_mass(eh, forced, tau)
        np.testing.assert_array_equal(kept_gpu, kept_ora)
        rp_o, ci_o = oracle.to_csr(kept_ora)
        np.testing.assert_array_equal(rp, rp_o)
        np.testing.assert_array_equal(ci[:rp[-1]], ci_o)
        mass_h = mass.cpu().numpy()
        np.testing.assert_allclose(mass_h, oracle.retained_mass(eh, kept_gpu), rtol=1e-12)
        # every row reaches tau unless it keeps everything (fixed-point rule; float sums agree
        # to far better than the slack used here)
        full = kept_gpu.all(axis=1)
        assert (mass_h[~full] >= tau - 1e-9).all()


def test_retained_mass_of_pooled_masks_against_oracle_energy():
    # retained mass of the pooled Top-K selection (the hot path's mask) measured with the GPU's
    # token-level energies, against the oracle's energies on the same mask
    m = dbsp()
    w = small_variants()["final_small"]
    say("case retained mass of pooled Top-K, final_small")
    q, k, _ = make_qkv(w, device="cuda", seed=6)
    idx = m.sparse_select(q, k, w.text, w.extra, density=w.param)
    e = m.block_energy(q, k)
    mass = m.retained_mass(e, idx, batch=w.batch, heads=w.heads)
    torch.cuda.synchronize()
    kept = P.csr_to_kept(idx.row_ptr.cpu().numpy().astype(np.int64),
                         idx.col_idx.cpu().numpy().astype(np.int64), w.n_k_blocks)
    e_ref = oracle.block_energy_rows(P.host(q), P.host(k), rows=range(w.rows))
    want = oracle.retained_mass(e_ref, kept)
    got = mass.cpu().numpy()
    assert np.abs(got - want).max() <= P.TOK_E_RTOL * 1.0 + kept.sum(axis=1).max() * P.TOK_E_ATOL
    # no block mask keeps more than the token-wise bound for its token budget
    ub = oracle.token_upper_bound(P.host(q), P.host(k), range(w.rows),
                                  (kept.sum(axis=1) * BLOCK).tolist())
    assert (got <= ub + 1e-4).all()


@pytest.mark.parametrize("name", ["star_mid_clip2", "dit_mass"])
def test_energy_full_size(name):
    # full size: every row sums to 1; sampled rows against the oracle
    w = WORKLOADS[name]
    say(f"case full {name} rows={w.rows} nkb={w.n_k_blocks}")
    q, k, _ = make_qkv(w, device="cuda", seed=0)
    e = dbsp().block_energy(q, k)
    torch.cuda.synchronize()
    eh = e.cpu().numpy().astype(np.float64)
    assert np.abs(eh.sum(axis=1) - 1.0).max() <= P.TOK_ROW_SUM
    rng = np.random.default_rng(1)
    rows = sorted(set([0, w.rows - 1] + rng.choice(w.rows, 4, replace=False).tolist()))
    qh, kh = P.host(q), P.host(k)
    P.check_token_energy(eh[rows], oracle.block_energy_rows(qh, kh, rows=rows))
