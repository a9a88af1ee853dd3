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
    # ... and keys shorter than one block (no whole block: only the partial-tile path runs),
    # with a partial query block too
    for lq, lk in ((128, 128), (128, 37 * 128), (5 * 128, 128), (200, 100), (300, 1000)):
        w = small_variants()["star_mid_small"].with_(heads=2, lq=lq, lk=lk)
        say(f"case edge lq={lq} lk={lk}")
        q, k, _ = make_qkv(w, device="cuda", seed=9)
        e = P.host(m.block_energy(q, k))
        torch.cuda.synchronize()
        e_ref = oracle.block_energy_rows(P.host(q), P.host(k), rows=range(w.rows))
        P.check_token_energy(e, e_ref)
        if w.n_k_blocks == 1:
            np.testing.assert_allclose(e, 1.0, rtol=0, atol=P.TOK_ROW_SUM)


def test_energy_deterministic():
    w = small_variants()["final_small"]
    say("case determinism final_small")
    q, k, _ = make_qkv(w, device="cuda", seed=2)
    a = dbsp().block_energy(q, k)
    b = dbsp().block_energy(q, k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_energy_workspace_slots():
    """The bf16 kernel runs one persistent workgroup per workspace slot (a slot holds a float per
    (key block, query) of the row in progress). Any number of slots gives the same bits: with one
    slot a single workgroup walks every row, reusing its slot and its LDS row after row; a
    ragged shape (partial last query and key blocks) checks the stale-slot case, where a row
    leaves entries the next row must not read."""
    m = dbsp()
    for name, lq, lk in (("final_small", None, None), ("star_mid_small", 1000, 2700)):
        w = small_variants()[name]
        if lq is not None:
            w = w.with_(lq=lq, lk=lk)
        say(f"case slots {name} Lq={w.lq} Lk={w.lk} rows={w.rows}")
        q, k, _ = make_qkv(w, device="cuda", seed=12)
        full = m.block_energy_workspace_bytes(q, k)
        slot = w.n_k_blocks * BLOCK * 4
        assert full == min(w.rows, 512) * slot
        e0, l0 = m.block_energy(q, k, return_lse=True)
        for n in (1, 2, 7, w.rows - 1):
            ws = torch.empty(n * slot + 100, dtype=torch.uint8, device="cuda")
            e1, l1 = m.block_energy(q, k, return_lse=True, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(e0, e1), n
            assert torch.equal(l0, l1), n
        e_ref = oracle.block_energy_rows(P.host(q), P.host(k), rows=range(w.rows))
        P.check_token_energy(P.host(e0), e_ref)
    q, k, _ = make_qkv(small_variants()["final_small"], device="cuda", seed=12)
    with pytest.raises(m.DbspError):
        m.block_energy(q, k, workspace=torch.empty(70 * BLOCK * 4 - 1, dtype=torch.uint8,
                                                   device="cuda"))


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


# one whole head (H / 2, batch 0) of each full-size workload against the oracle, row by row;
# the DiT head (591 query blocks against 75,648 keys each) is checked in three parts so that
# each part stays well inside the per-test time limit
FULL_HEAD_PARTS = [("star_mid_clip2", 0, 1), ("dit_mass", 0, 3), ("dit_mass", 1, 3),
                   ("dit_mass", 2, 3)]


@pytest.mark.parametrize("name,part,parts", FULL_HEAD_PARTS)
def test_energy_full_size(name, part, parts):
    # full size: every row of every head sums to 1; one whole head against the oracle
    w = WORKLOADS[name]
    say(f"case full {name} rows={w.rows} nkb={w.n_k_blocks} head part {part + 1}/{parts}")
    q, k, _ = make_qkv(w, device="cuda", seed=0)
    e = dbsp().block_energy(q, k)
    torch.cuda.synchronize()
    eh = e.cpu().numpy().astype(np.float64)
    assert np.abs(eh.sum(axis=1) - 1.0).max() <= P.TOK_ROW_SUM
    h = w.heads // 2
    nqb = w.n_q_blocks
    lo, hi = part * nqb // parts, (part + 1) * nqb // parts
    qh, kh = P.host(q[0:1, h:h + 1]), P.host(k[0:1, h:h + 1])
    P.check_token_energy(eh[h * nqb + lo:h * nqb + hi],
                         oracle.block_energy_rows(qh, kh, rows=range(lo, hi)))
    say(f"  head {h} query blocks [{lo}, {hi}) match the oracle")


def test_select_energy_unnormalised_rows():
    # rows that do not sum to 1 but stay inside the documented range (values in [0, 1], row sums
    # at most 2): sums up to 2, sums below tau (every block kept), single dominant blocks, and
    # exact ties; masks bit-exact against the oracle on the same float32 values
    m = dbsp()
    rng = np.random.default_rng(61)
    batch, heads, nqb, nkb = 1, 2, 40, 300
    rows = batch * heads * nqb
    p = rng.random((rows, nkb)) ** 4
    target = rng.uniform(0.3, 1.95, size=(rows, 1))
    p = p / p.sum(axis=1, keepdims=True) * target
    p[0] = 1.99 / nkb                                  # all tied, sum 1.99
    p[1] = 0.0
    p[1, 7] = 1.0                                      # one block holds everything
    p[1, 8] = 1.0                                      # ... and a tie at the top: sum 2
    p[2] = 0.5 / nkb                                   # sum 0.5: never reaches tau
    p = np.minimum(p, 1.0).astype(np.float32)
    # keep every float32 row sum (rounded up) within 2
    assert (p.astype(np.float64).sum(axis=1) <= 2.0).all()
    e = torch.from_numpy(p).cuda()
    forced = oracle.forced_blocks(nkb, (0, 2), (0, 0))
    say(f"case un-normalised rows: rows={rows} nkb={nkb}")
    for tau in (0.25, 0.9, 0.999):
        idx = m.select_energy(e, tau, (0, 2), (0, 0), batch=batch, heads=heads)
        torch.cuda.synchronize()
        rp = idx.row_ptr.cpu().numpy().astype(np.int64)
        ci = idx.col_idx.cpu().numpy().astype(np.int64)
        kept_gpu = P.csr_to_kept(rp, ci, nkb)
        kept_ora = oracle.select_mass(p.astype(np.float64), forced, tau)
        np.testing.assert_array_equal(kept_gpu, kept_ora)
        if tau > 0.5:
            assert kept_gpu[2].all()                   # row 2 never reaches tau
