"""GPU parity of the cross-input vote (CalibAtt Eq. (8)/(9)) and of the offline calibration
pipeline it closes: per-input token-level energies -> per-input masks at tau -> vote at rho ->
one static CSR, reused by the sparse attention on a new input.

Bars: counts and voted masks bit-exact against the oracle (integer counts, exact rational
comparison); per-input masks bit-exact against the oracle selecting from the GPU's energies;
attention with the static CSR at the bf16 bar of the hot path.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from synth import BLOCK, make_qkv, small_variants
from tests import parity as P

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "vote_example.json")


def dbsp():
    import dynamic_block_sparse_pool_amd as m
    return m


def say(msg):
    print(f"[gpu-vote] {msg}", flush=True)


def index_of(kept: np.ndarray, nqb: int, dev="cuda"):
    m = dbsp()
    rp, ci = oracle.to_csr(kept)
    return m.BlockIndex(torch.from_numpy(rp.astype(np.int32)).to(dev),
                        torch.from_numpy(np.maximum(ci, 0).astype(np.int32) if ci.size else
                                         np.zeros(1, np.int32)).to(dev),
                        nqb, kept.shape[1], None)


def voted(vote, rho, nkb):
    idx = vote.select(rho)
    torch.cuda.synchronize()
    return P.csr_to_kept(idx.row_ptr.cpu().numpy().astype(np.int64),
                         idx.col_idx.cpu().numpy().astype(np.int64), nkb)


def test_vote_worked_example():
    g = json.load(open(GOLDEN))
    say("case worked example: 64 inputs, rho 0.5")
    counts = np.array(g["counts"])
    nkb = counts.size
    vote = dbsp().MaskVote(1, 1, 1, nkb, "cuda")
    for p in range(g["n_inputs"]):
        vote.add(index_of((p < counts)[None, :], 1))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(vote.counts.cpu().numpy()[0], counts)
    assert voted(vote, g["rho"], nkb)[0].tolist() == g["kept"]


def test_vote_random_masks():
    rng = np.random.default_rng(17)
    batch, heads, nqb, nkb, n = 1, 2, 3, 70, 13
    rows = batch * heads * nqb
    say(f"case random masks rows={rows} nkb={nkb} inputs={n}")
    masks = rng.random((n, rows, nkb)) < rng.random((1, rows, nkb))
    masks[:, :, 0] = True
    vote = dbsp().MaskVote(batch, heads, nqb, nkb, "cuda")
    for p in range(n):
        vote.add(index_of(masks[p], nqb))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(vote.counts.cpu().numpy(), masks.sum(axis=0))
    for rho in (0.0, 0.3, 1 / 3, 0.5, 12 / 13, 1.0):
        np.testing.assert_array_equal(voted(vote, rho, nkb), oracle.vote_masks(masks, rho))


def test_calibration_pipeline_and_static_reuse():
    m = dbsp()
    w = small_variants()["dit_mass_small"]
    nkb, nqb = w.n_k_blocks, w.n_q_blocks
    tau, rho, n = 0.9, 0.5, 8
    forced = oracle.forced_blocks(nkb, w.text, w.extra)
    vote = m.MaskVote(w.batch, w.heads, nqb, nkb, "cuda")
    masks = []
    for p in range(n):
        say(f"case calibration input {p}")
        q, k, _ = make_qkv(w, device="cuda", seed=100 + p)
        e = m.block_energy(q, k)
        idx = m.select_energy(e, tau, w.text, w.extra, batch=w.batch, heads=w.heads)
        vote.add(idx)
        torch.cuda.synchronize()
        kept = P.csr_to_kept(idx.row_ptr.cpu().numpy().astype(np.int64),
                             idx.col_idx.cpu().numpy().astype(np.int64), nkb)
        np.testing.assert_array_equal(kept, oracle.select_mass(P.host(e), forced, tau))
        masks.append(kept)
    static = vote.select(rho)
    torch.cuda.synchronize()
    kept_static = P.csr_to_kept(static.row_ptr.cpu().numpy().astype(np.int64),
                                static.col_idx.cpu().numpy().astype(np.int64), nkb)
    np.testing.assert_array_equal(kept_static, oracle.vote_masks(np.stack(masks), rho))
    # the static CSR drives the attention of a new input
    say("case static CSR reused on a new input")
    q, k, v = make_qkv(w, device="cuda", seed=999)
    o, lse = m.sparse_attn_fwd(q, k, v, static, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    rp = static.row_ptr.cpu().numpy().astype(np.int64)
    ci = static.col_idx.cpu().numpy().astype(np.int64)
    o_ref, lse_ref = oracle.attention_rows(P.host(q), P.host(k), P.host(v), rp, ci)
    P.check_attention(P.host(o).reshape(o_ref.shape), P.host(lse).reshape(lse_ref.shape), o_ref,
                      lse_ref, bf16_inputs=True)
