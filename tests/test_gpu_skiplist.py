"""GPU parity of the interval skip list (CalibAtt key design 4): CSR -> maximal runs -> CSR,
bit-exact against the oracle's encoding, on the hot path's own masks and on random masks."""
import numpy as np
import pytest
import torch

import oracle
from synth import BLOCK, make_qkv, small_variants
from tests import parity as P

pytestmark = pytest.mark.gpu


def dbsp():
    import dynamic_block_sparse_pool_amd as m
    return m


def say(msg):
    print(f"[gpu-skiplist] {msg}", flush=True)


def check_round_trip(index, kept, batch, heads, nqb, nkb):
    m = dbsp()
    iv_ptr, iv = m.to_intervals(index, batch, heads)
    back = m.from_intervals(iv_ptr, iv, nqb, nkb, batch, heads)
    torch.cuda.synchronize()
    ptr_ref, iv_ref = oracle.to_intervals(kept)
    ptr = iv_ptr.cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(ptr, ptr_ref)
    np.testing.assert_array_equal(iv.cpu().numpy()[:ptr[-1]].astype(np.int64), iv_ref)
    rp = back.row_ptr.cpu().numpy().astype(np.int64)
    ci = back.col_idx.cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(P.csr_to_kept(rp, ci, nkb), kept)
    np.testing.assert_array_equal(rp, index.row_ptr.cpu().numpy())
    return int(ptr[-1])


@pytest.mark.parametrize("name", ["final_small", "clip1_small", "dit_mass_small"])
def test_intervals_of_selected_masks(name):
    m = dbsp()
    w = small_variants()[name]
    say(f"case {name}")
    q, k, _ = make_qkv(w, device="cuda", seed=51)
    kw = dict(density=w.param) if w.mode == "topk" else dict(mass=w.param)
    idx = m.sparse_select(q, k, w.text, w.extra, **kw)
    torch.cuda.synchronize()
    kept = P.csr_to_kept(idx.row_ptr.cpu().numpy().astype(np.int64),
                         idx.col_idx.cpu().numpy().astype(np.int64), w.n_k_blocks)
    runs = check_round_trip(idx, kept, w.batch, w.heads, w.n_q_blocks, w.n_k_blocks)
    say(f"  {int(kept.sum())} kept blocks in {runs} runs")


def test_intervals_random_and_extreme_masks():
    rng = np.random.default_rng(52)
    batch, heads, nqb, nkb = 1, 3, 5, 131
    rows = batch * heads * nqb
    say(f"case random masks rows={rows} nkb={nkb}")
    kept = rng.random((rows, nkb)) < rng.random((rows, 1))
    kept[0] = False                          # empty row
    kept[1] = True                           # one run over everything
    kept[2] = np.arange(nkb) % 2 == 0        # the most runs a row can have
    rp, ci = oracle.to_csr(kept)
    m = dbsp()
    idx = m.BlockIndex(torch.from_numpy(rp.astype(np.int32)).cuda(),
                       torch.from_numpy(ci.astype(np.int32)).cuda(), nqb, nkb, None)
    check_round_trip(idx, kept, batch, heads, nqb, nkb)


def test_intervals_skip_out_of_range_neighbours():
    # rows of an ascending CSR that also hold out-of-range entries next to the range ends: a -1
    # right before block 0 and nkb right after block nkb - 1 must neither join nor split a run,
    # so the encoding equals the oracle's encoding of the in-range mask (the kernels skip
    # out-of-range entries)
    nkb = 11
    rows_cols = [
        [-1, 0, 1, 2, 6, nkb - 1, nkb],
        [-5, -1, 0],
        [nkb - 1, nkb, nkb + 3],
        [-1],
        [nkb],
        [-1, 0, nkb - 2, nkb - 1, nkb],
        [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11],
        [],
    ]
    batch, heads, nqb = 1, 1, len(rows_cols)
    rp = np.zeros(nqb + 1, np.int64)
    np.cumsum([len(r) for r in rows_cols], out=rp[1:])
    ci = np.array([c for r in rows_cols for c in r], np.int64)
    kept = np.zeros((nqb, nkb), bool)
    for r, cols in enumerate(rows_cols):
        for c in cols:
            if 0 <= c < nkb:
                kept[r, c] = True
    say(f"case out-of-range neighbours: rows={nqb} nkb={nkb} entries={ci.size}")
    m = dbsp()
    idx = m.BlockIndex(torch.from_numpy(rp.astype(np.int32)).cuda(),
                       torch.from_numpy(ci.astype(np.int32)).cuda(), nqb, nkb, None)
    iv_ptr, iv = m.to_intervals(idx, batch, heads)
    back = m.from_intervals(iv_ptr, iv, nqb, nkb, batch, heads)
    torch.cuda.synchronize()
    ptr_ref, iv_ref = oracle.to_intervals(kept)
    ptr = iv_ptr.cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(ptr, ptr_ref)
    np.testing.assert_array_equal(iv.cpu().numpy()[:ptr[-1]].astype(np.int64), iv_ref)
    brp = back.row_ptr.cpu().numpy().astype(np.int64)
    bci = back.col_idx.cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(P.csr_to_kept(brp, bci, nkb), kept)
