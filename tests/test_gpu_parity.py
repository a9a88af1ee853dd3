"""GPU parity: the HIP path (through the C ABI) against the oracle on the same seeded inputs.

Bars: pooled scores within 1e-3 relative (cancellation floor, see tests/parity.py); masks
bit-exact when the oracle selects from the very scores the GPU compared (S in Top-K mode, p in
mass mode); where they differ from the oracle's own masks, only at near ties; O within 1e-5
max abs for fp32 inputs, 2e-2 max / 2e-3 mean abs for bf16 inputs (fp64 oracle on the
bf16-rounded values); lse alongside.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import BLOCK, WORKLOADS, Workload, make_qkv, small_variants
from tests import parity as P

pytestmark = pytest.mark.gpu


def dbsp():
    import dynamic_block_sparse_pool_amd as m
    return m


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)


def run_path(w: Workload, q, k, v, out_dtype=torch.float32, out=None, **kw):
    m = dbsp()
    if w.mode == "topk":
        idx = m.sparse_select(q, k, w.text, w.extra, density=w.param, return_scores=True, **kw)
    else:
        idx = m.sparse_select(q, k, w.text, w.extra, mass=w.param, return_scores=True, **kw)
    o, lse = m.sparse_attn_fwd(q, k, v, idx, out_dtype=out_dtype, return_lse=True, out=out)
    torch.cuda.synchronize()
    return idx, o, lse


def oracle_select_on(w: Workload, scores2d: np.ndarray, forced: np.ndarray, topk_override=None):
    if w.mode == "topk":
        kk = (oracle.topk_budget(w.param, int((~forced).sum())) if topk_override is None
              else topk_override)
        return oracle.select_topk(scores2d, forced, kk)
    return oracle.select_mass(scores2d, forced, w.param)


def full_check_small(w: Workload, seed=3, inputs=None, score_scale=None, out=None, attention=True):
    """Selection and attention of workload w through the C ABI against the oracle on the same
    values: every score, every mask row and CSR entry, every output and lse. `inputs` may be
    strided views and `out` a strided fp32 output view (the oracle reads their values);
    attention=False stops after the selection checks."""
    say(f"case {w.name} B={w.batch} H={w.heads} Lq={w.lq} Lk={w.lk} d={w.head_dim} {w.dtype} "
        f"{w.mode}={w.param} seed={seed}")
    q, k, v = inputs if inputs is not None else make_qkv(w, device="cuda", seed=seed)
    kw = {} if score_scale is None else {"score_scale": score_scale}
    idx, o, lse = run_path(w, q, k, v, out=out, **kw)
    qh, kh, vh = P.host(q), P.host(k), P.host(v)
    ref = oracle.sparse_select(qh, kh, w.text, w.extra, w.mode, w.param, score_scale=score_scale)
    nkb, nqb = w.n_k_blocks, w.n_q_blocks
    forced = ref["forced"]
    scores = P.host(idx.scores)
    scale = score_scale or 1.0 / math.sqrt(w.head_dim)
    if w.mode == "topk":
        s4 = scores.reshape(w.batch, w.heads, nqb, nkb)
        for b in range(w.batch):
            for h in range(w.heads):
                P.check_scores(s4[b, h], ref["qbar"][b, h], ref["kbar"][b, h], scale)
    else:
        P.check_energies(scores, ref["scores"].reshape(-1, nkb))
    rp = idx.row_ptr.cpu().numpy().astype(np.int64)
    ci = idx.col_idx.cpu().numpy().astype(np.int64)
    kept_gpu = P.csr_to_kept(rp, ci, nkb)
    kept_ora = oracle_select_on(w, scores, forced)
    np.testing.assert_array_equal(kept_gpu, kept_ora)
    rp_ora, ci_ora = oracle.to_csr(kept_ora)
    np.testing.assert_array_equal(rp, rp_ora)
    np.testing.assert_array_equal(ci[:rp[-1]], ci_ora)
    if w.mode == "topk":
        bound = (np.linalg.norm(ref["qbar"], axis=-1)[..., :, None]
                 * np.linalg.norm(ref["kbar"], axis=-1)[..., None, :] * scale)
        s_ref = ref["scores"]
        tol = (P.SCORE_RTOL * np.maximum(np.abs(s_ref), P.SCORE_FLOOR * bound)).reshape(-1, nkb)
        ndiff = P.topk_near_tie_ok(kept_gpu, ref["kept"].reshape(-1, nkb),
                                   s_ref.reshape(-1, nkb), forced, tol)
        say(f"  rows differing from the oracle's own masks (near ties only): {ndiff}")
    if not attention:
        return idx, o, lse
    o_ref, lse_ref = oracle.attention_rows(qh, kh, vh, rp, ci, scale=1.0 / math.sqrt(w.head_dim))
    o_ref, lse_ref = P.rows_to_tokens(o_ref, lse_ref, w.batch, w.heads, w.lq)
    mx, mean = P.check_attention(P.host(o), P.host(lse), o_ref, lse_ref, w.dtype == "bf16")
    say(f"  O max err {mx:.2e} mean {mean:.2e}; nnz {int(rp[-1])}")
    return idx, o, lse


@pytest.mark.parametrize("name", list(small_variants()))
def test_small_workloads(name):
    full_check_small(small_variants()[name])


def test_toy_density_one_equals_dense():
    w = WORKLOADS["toy_dense"]
    q, k, v = make_qkv(w, device="cuda", seed=0)
    idx, o, lse = run_path(w, q, k, v)
    assert idx.nnz() == w.rows * w.n_k_blocks
    od, lsed = oracle.attention_dense(P.host(q), P.host(k), P.host(v))
    assert np.abs(P.host(o) - od).max() <= P.F32_O_MAX
    assert np.abs(P.host(lse) - lsed).max() <= P.F32_LSE


def test_bf16_density_one_equals_dense():
    w = small_variants()["star_mid_small"].with_(param=1.0, text=(0, 0))
    q, k, v = make_qkv(w, device="cuda", seed=8)
    idx, o, lse = run_path(w, q, k, v)
    assert idx.nnz() == w.rows * w.n_k_blocks
    od, lsed = oracle.attention_dense(P.host(q), P.host(k), P.host(v))
    P.check_attention(P.host(o), P.host(lse), od, lsed, True)


def test_adversarial_ties():
    # Integer-valued tokens, constant inside each block: pooled scores are small integers over
    # sqrt(d) and tie massively. The GPU's tie-breaking must equal the oracle's.
    w = small_variants()["final_small"].with_(name="ties")
    g = torch.Generator(device="cuda").manual_seed(77)
    def blocky(length):
        nb = length // BLOCK
        c = torch.randint(-1, 2, (w.batch, w.heads, nb, 1, w.head_dim), generator=g, device="cuda")
        return c.expand(-1, -1, -1, BLOCK, -1).reshape(w.batch, w.heads, length, w.head_dim) \
            .to(torch.bfloat16).contiguous()
    q, k = blocky(w.lq), blocky(w.lk)
    v = make_qkv(w, device="cuda", seed=1)[2]
    full_check_small(w, inputs=(q, k, v))
    wm = small_variants()["dit_mass_small"].with_(name="ties_mass", param=0.6)
    qm, km = (torch.randint(-1, 2, (1, 2, wm.lq, wm.head_dim), generator=g, device="cuda")
              .to(torch.bfloat16) for _ in range(2))
    vm = make_qkv(wm, device="cuda", seed=1)[2]
    full_check_small(wm, inputs=(qm.contiguous(), km.contiguous(), vm))


def test_topk_scores_over_many_magnitudes():
    # Key blocks scaled by powers of two (2^-12 .. 2^11): the pooled scores of a row spread over
    # many exponents, so the threshold's top byte is settled by the ballot walk at low density
    # and by the histogram after the walk gives up at high density. Masks must equal the
    # oracle's on the GPU's scores either way. Selection only: logits reach ~1e4 here, beyond
    # the range the attention tolerances are derived for.
    for density in (0.1875, 0.625):
        w = small_variants()["star_mid_small"].with_(name=f"magnitudes_{density}", heads=2,
                                                       param=density)
        q, k, v = make_qkv(w, device="cuda", seed=21)
        nb = w.lk // BLOCK
        scale = torch.tensor([2.0 ** ((j * 7) % 24 - 12) for j in range(nb)], device="cuda")
        ks = (k.float().reshape(1, w.heads, nb, BLOCK, w.head_dim) * scale[:, None, None])
        k2 = ks.reshape(k.shape).to(torch.bfloat16).contiguous()
        full_check_small(w, inputs=(q, k2, v), attention=False)


def test_all_equal_scores_keep_lowest_indices():
    w = small_variants()["star_mid_small"].with_(name="flat")
    q = torch.ones((1, w.heads, w.lq, w.head_dim), device="cuda", dtype=torch.bfloat16)
    k = torch.ones((1, w.heads, w.lk, w.head_dim), device="cuda", dtype=torch.bfloat16)
    v = make_qkv(w, device="cuda", seed=2)[2]
    idx, _, _ = full_check_small(w, inputs=(q, k, v))
    forced = oracle.forced_blocks(w.n_k_blocks, w.text, w.extra)
    kk = oracle.topk_budget(w.param, int((~forced).sum()))
    want = list(range(w.text[1])) + list(range(w.text[1], w.text[1] + kk))
    rp = idx.row_ptr.cpu().numpy()
    ci = idx.col_idx.cpu().numpy()
    for r in range(w.rows):
        assert ci[rp[r]:rp[r + 1]].tolist() == want


def test_edge_cases():
    base = small_variants()["star_mid_small"]
    cases = [
        base.with_(name="density0_no_forced", text=(0, 0), param=0.0),       # empty rows
        base.with_(name="density0_forced", param=0.0),                        # forced only
        base.with_(name="all_forced", text=(0, 10), extra=(10, 22), param=0.5),  # no candidates
        base.with_(name="one_key_block", lk=BLOCK, text=(0, 0), param=1.0),
        base.with_(name="one_query_block", lq=BLOCK),
        base.with_(name="two_forced_ranges", text=(0, 2), extra=(5, 9), param=0.3),
        base.with_(name="mass_tau_one", mode="mass", param=1.0, text=(0, 0)),
        base.with_(name="mass_with_forced", mode="mass", param=0.7, text=(0, 2), extra=(3, 4)),
        base.with_(name="mass_low_tau", mode="mass", param=0.05),
        base.with_(name="fp32_d128", dtype="f32", structure="iid"),
        WORKLOADS["toy"].with_(name="toy_mass", mode="mass", param=0.5),
    ]
    for w in cases:
        full_check_small(w, seed=5)


def test_empty_rows_output_zero():
    w = small_variants()["star_mid_small"].with_(text=(0, 0), param=0.0)
    q, k, v = make_qkv(w, device="cuda", seed=1)
    idx, o, lse = run_path(w, q, k, v)
    assert idx.nnz() == 0
    assert (o == 0).all().item() and torch.isneginf(lse).all().item()


def test_explicit_scales():
    w = small_variants()["final_small"]
    full_check_small(w, score_scale=0.05)
    q, k, v = make_qkv(w, device="cuda", seed=4)
    m = dbsp()
    idx = m.sparse_select(q, k, w.text, w.extra, density=w.param)
    o, lse = m.sparse_attn_fwd(q, k, v, idx, softmax_scale=0.02, out_dtype=torch.float32,
                               return_lse=True)
    torch.cuda.synchronize()
    rp = idx.row_ptr.cpu().numpy().astype(np.int64)
    ci = idx.col_idx.cpu().numpy().astype(np.int64)
    o_ref, lse_ref = oracle.attention_rows(P.host(q), P.host(k), P.host(v), rp, ci, scale=0.02)
    P.check_attention(P.host(o).reshape(o_ref.shape), P.host(lse).reshape(lse_ref.shape), o_ref,
                      lse_ref, True)


def test_topk_override():
    w = small_variants()["clip1_small"]
    q, k, v = make_qkv(w, device="cuda", seed=6)
    idx = dbsp().sparse_select(q, k, w.text, w.extra, density=0.0, topk_override=3,
                               return_scores=True)
    torch.cuda.synchronize()
    forced = oracle.forced_blocks(w.n_k_blocks, w.text, w.extra)
    kept = P.csr_to_kept(idx.row_ptr.cpu().numpy(), idx.col_idx.cpu().numpy(), w.n_k_blocks)
    want = oracle.select_topk(P.host(idx.scores), forced, 3)
    np.testing.assert_array_equal(kept, want)


def test_max_key_blocks():
    w = WORKLOADS["final_720p_clip2"].with_(name="max_nkb", heads=1, lq=2 * BLOCK,
                                             lk=2048 * BLOCK)
    full_check_small(w, seed=9)
    wm = w.with_(name="max_nkb_mass", mode="mass", param=0.9)
    full_check_small(wm, seed=9)


@pytest.mark.parametrize("lk", [2100 * BLOCK, 2100 * BLOCK - 50])
def test_rows_longer_than_one_staging_window(lk):
    # density 1: every row keeps all 2,100 key blocks, more than one LDS staging window of the
    # attention kernel holds (2,048), so each row's list is staged and streamed in two windows;
    # the ragged case also sends the partial last block through its own path after them
    w = WORKLOADS["final_720p_clip2"].with_(name="two_windows", heads=1, lq=2 * BLOCK, lk=lk,
                                             param=1.0, text=(0, 0))
    # (selection stops at 2,048 key blocks; the attention takes any CSR, built here directly)
    m = dbsp()
    say(f"case two_windows: Lq={w.lq} Lk={w.lk}")
    q, k, v = make_qkv(w, device="cuda", seed=12)
    nkb = w.n_k_blocks
    row_ptr = torch.arange(0, (w.rows + 1) * nkb, nkb, dtype=torch.int32, device="cuda")
    col_idx = torch.arange(nkb, dtype=torch.int32, device="cuda").repeat(w.rows)
    idx = m.BlockIndex(row_ptr=row_ptr, col_idx=col_idx, n_q_blocks=w.n_q_blocks, n_k_blocks=nkb)
    o, lse = m.sparse_attn_fwd(q, k, v, idx, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    od, lsed = oracle.attention_dense(P.host(q), P.host(k), P.host(v))
    P.check_attention(P.host(o), P.host(lse), od, lsed, True)


def test_bf16_d64_select():
    w = small_variants()["star_mid_small"].with_(name="bf16_d64", head_dim=64)
    q, k, _ = make_qkv(w, device="cuda", seed=2)
    idx = dbsp().sparse_select(q, k, w.text, w.extra, density=w.param, return_scores=True)
    torch.cuda.synchronize()
    ref = oracle.sparse_select(P.host(q), P.host(k), w.text, w.extra, "topk", w.param)
    s = P.host(idx.scores).reshape(1, w.heads, w.n_q_blocks, w.n_k_blocks)
    for h in range(w.heads):
        P.check_scores(s[0, h], ref["qbar"][0, h], ref["kbar"][0, h], 1 / math.sqrt(64))
    kept = P.csr_to_kept(idx.row_ptr.cpu().numpy(), idx.col_idx.cpu().numpy(), w.n_k_blocks)
    np.testing.assert_array_equal(kept, oracle_select_on(w, s.reshape(-1, w.n_k_blocks),
                                                         ref["forced"]))


def test_deterministic():
    w = small_variants()["final_small"]
    q, k, v = make_qkv(w, device="cuda", seed=11)
    a_idx, a_o, a_l = run_path(w, q, k, v, out_dtype=torch.bfloat16)
    b_idx, b_o, b_l = run_path(w, q, k, v, out_dtype=torch.bfloat16)
    assert torch.equal(a_idx.row_ptr, b_idx.row_ptr)
    assert torch.equal(a_idx.col_idx[:a_idx.nnz()], b_idx.col_idx[:b_idx.nnz()])
    assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)


def test_bf16_output_rounds_fp32_output():
    w = small_variants()["clip1_small"]
    q, k, v = make_qkv(w, device="cuda", seed=12)
    idx, o32, _ = run_path(w, q, k, v, out_dtype=torch.float32)
    o16 = dbsp().sparse_attn_fwd(q, k, v, idx, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))


@pytest.mark.parametrize("mode", ["topk", "mass"])
def test_forced_list(mode):
    # an explicit, scattered forced list (across bitmask words, unsorted) instead of ranges:
    # masks bit-exact against the oracle selecting with that forced set from the GPU's scores
    m = dbsp()
    w = small_variants()["final_small"].with_(lk=(4 + 65 + 65) * BLOCK)
    nkb = w.n_k_blocks
    forced_list = [130, 0, 64, 63, 7, 101]
    say(f"case forced list {forced_list} mode={mode} nkb={nkb}")
    q, k, _ = make_qkv(w, device="cuda", seed=21)
    kw = dict(density=0.2) if mode == "topk" else dict(mass=0.8)
    idx = m.sparse_select(q, k, density=kw.get("density"), mass=kw.get("mass"),
                          return_scores=True, forced_blocks=forced_list)
    torch.cuda.synchronize()
    forced = np.zeros(nkb, dtype=bool)
    forced[forced_list] = True
    scores = P.host(idx.scores)
    if mode == "topk":
        kk = oracle.topk_budget(0.2, int((~forced).sum()))
        kept_ora = oracle.select_topk(scores, forced, kk)
    else:
        kept_ora = oracle.select_mass(scores, forced, 0.8)
    rp = idx.row_ptr.cpu().numpy().astype(np.int64)
    ci = idx.col_idx.cpu().numpy().astype(np.int64)
    kept_gpu = P.csr_to_kept(rp, ci, nkb)
    np.testing.assert_array_equal(kept_gpu, kept_ora)
    assert kept_gpu[:, forced_list].all()
    # the list equal to a range gives the range's result bit for bit
    idx_r = m.sparse_select(q, k, (0, 4), density=kw.get("density"), mass=kw.get("mass"))
    idx_l = m.sparse_select(q, k, density=kw.get("density"), mass=kw.get("mass"),
                            forced_blocks=[3, 2, 1, 0])
    torch.cuda.synchronize()
    n = idx_r.nnz()
    assert n == idx_l.nnz()
    assert torch.equal(idx_r.row_ptr, idx_l.row_ptr)
    assert torch.equal(idx_r.col_idx[:n], idx_l.col_idx[:n])



PARTIAL = {
    # lengths that are not multiples of 128: partial last query and key blocks
    "bf16 topk": small_variants()["final_small"].with_(name="partial_topk",
                                                       lq=17 * BLOCK - 37, lk=70 * BLOCK - 51),
    "bf16 mass": small_variants()["dit_mass_small"].with_(name="partial_mass",
                                                          lq=19 * BLOCK - 48, lk=19 * BLOCK - 48),
    "bf16 clip1": small_variants()["clip1_small"].with_(name="partial_clip1",
                                                        lq=11 * BLOCK - 1, lk=23 * BLOCK - 127),
    "fp32 toy": WORKLOADS["toy"].with_(name="partial_toy", lq=1000, lk=900),
    "bf16 one short block": small_variants()["star_mid_small"].with_(
        name="partial_tiny", lq=77, lk=100, text=(0, 1)),
}


@pytest.mark.parametrize("name", list(PARTIAL))
def test_partial_blocks(name):
    full_check_small(PARTIAL[name], seed=31)


def test_partial_blocks_energy_and_anchor():
    m = dbsp()
    w = PARTIAL["bf16 mass"]
    say(f"case partial energy lq={w.lq} lk={w.lk}")
    q, k, v = make_qkv(w, device="cuda", seed=32)
    e, lse = m.block_energy(q, k, return_lse=True)
    torch.cuda.synchronize()
    qh, kh = P.host(q), P.host(k)
    P.check_token_energy(P.host(e), oracle.block_energy_rows(qh, kh, rows=range(w.rows)))
    assert np.abs(P.host(lse) - oracle.attention_dense(qh, kh, kh)[1]).max() <= P.TOK_LSE
    wf = PARTIAL["fp32 toy"]
    say(f"case partial energy fp32 lq={wf.lq} lk={wf.lk}")
    qf, kf, _ = make_qkv(wf, device="cuda", seed=33)
    ef = m.block_energy(qf, kf)
    torch.cuda.synchronize()
    P.check_token_energy(P.host(ef), oracle.block_energy_rows(P.host(qf), P.host(kf),
                                                              rows=range(wf.rows)))
    # anchor path with keys ending in a partial block
    say("case partial anchor")
    o, l2 = m.anchor_attn_fwd(q, k, v, 3, 7, 100, 2, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.anchor_attention(qh, kh, P.host(v), 3, 7, 100, 2)
    P.check_attention(P.host(o), P.host(l2), o_ref, l_ref, bf16_inputs=True)


def test_batch_two():
    # two batch entries: rows (b * H + h) * nQB + i, per-(b, h) pooling and K/V bases
    w = small_variants()["final_small"].with_(name="batch2", batch=2, heads=3,
                                              lq=7 * BLOCK, lk=(4 + 20) * BLOCK)
    full_check_small(w, seed=61)
    wm = small_variants()["dit_mass_small"].with_(name="batch2_mass", batch=2,
                                                  lq=5 * BLOCK - 3, lk=9 * BLOCK - 100)
    full_check_small(wm, seed=62)
