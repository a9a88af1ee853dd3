"""Longest-first row order for the attention launch: the order is a permutation of the rows, heads
in order, each head's rows with non-increasing kept counts (equal counts in any order), and
attention started in that order gives bit-identical O and lse to attention started in row order
(each row is computed by one workgroup with the same instructions whichever workgroup that is)."""
import numpy as np
import pytest
import torch

from synth import BLOCK, make_qkv, small_variants

pytestmark = pytest.mark.gpu


def dbsp():
    import dynamic_block_sparse_pool_amd as m
    return m


def say(msg):
    print(f"[gpu-order] {msg}", flush=True)


@pytest.mark.parametrize("name,lq", [("dit_mass_small", None), ("dit_mass_small", 19 * BLOCK - 48)])
def test_lpt_order_and_ordered_attention(name, lq):
    m = dbsp()
    w = small_variants()[name]
    if lq is not None:
        w = w.with_(lq=lq, lk=lq)
    say(f"case {name}: B={w.batch} H={w.heads} Lq={w.lq} Lk={w.lk} mass={w.param}")
    q, k, v = make_qkv(w, device="cuda", seed=81)
    idx = m.sparse_select(q, k, w.text, w.extra, mass=w.param)
    order = m.lpt_order(q, k, idx)
    torch.cuda.synchronize()
    rp = idx.row_ptr.cpu().numpy().astype(np.int64)
    counts = rp[1:] - rp[:-1]
    o = order.cpu().numpy()
    assert np.array_equal(np.sort(o), np.arange(idx.rows))          # a permutation
    nqb = idx.n_q_blocks
    head = o // nqb
    assert (np.diff(head) >= 0).all()                                # heads in order
    for hh in np.unique(head):
        assert (np.diff(counts[o[head == hh]]) <= 0).all()           # longest first per head
    assert len(np.unique(counts)) > 1                                # the case has unequal rows
    o1, l1 = m.sparse_attn_fwd(q, k, v, idx, out_dtype=torch.float32, return_lse=True)
    o2, l2 = m.sparse_attn_fwd(q, k, v, idx, out_dtype=torch.float32, return_lse=True,
                               row_order=order)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_reversed_order_and_out_of_range_entries():
    # any permutation gives the same result; entries outside [0, rows) leave their slot idle
    m = dbsp()
    w = small_variants()["final_small"]
    say(f"case final_small reversed / out-of-range: H={w.heads} Lq={w.lq}")
    q, k, v = make_qkv(w, device="cuda", seed=82)
    idx = m.sparse_select(q, k, w.text, w.extra, density=w.param)
    rows = idx.rows
    rev = torch.arange(rows - 1, -1, -1, dtype=torch.int32, device="cuda")
    o1 = m.sparse_attn_fwd(q, k, v, idx, out_dtype=torch.float32)
    o2 = m.sparse_attn_fwd(q, k, v, idx, out_dtype=torch.float32, row_order=rev)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    # drop the last row from the order: its output keeps the value it had before the call
    part = rev.clone()
    part[0] = rows + 5                                               # out of range: skipped
    o3 = torch.full_like(o1, 7.0)
    m.sparse_attn_fwd(q, k, v, idx, out_dtype=torch.float32, row_order=part, out=o3)
    torch.cuda.synchronize()
    nqb = idx.n_q_blocks
    last = rows - 1
    b_h, i = divmod(last, nqb)
    bb, hh = divmod(b_h, w.heads)
    untouched = o3[bb, hh, i * BLOCK:(i + 1) * BLOCK]
    assert torch.all(untouched == 7.0)
    mask = torch.ones_like(o1, dtype=torch.bool)
    mask[bb, hh, i * BLOCK:(i + 1) * BLOCK] = False
    assert torch.equal(o3[mask], o1[mask])


def test_index_on_the_host_is_rejected():
    # a CSR left in host memory must be refused before any launch (the kernels would read
    # host addresses)
    m = dbsp()
    w = small_variants()["star_mid_small"]
    q, k, v = make_qkv(w, device="cuda", seed=4)
    idx = m.sparse_select(q, k, w.text, w.extra, density=w.param)
    host = m.BlockIndex(idx.row_ptr.cpu(), idx.col_idx.cpu(), idx.n_q_blocks, idx.n_k_blocks)
    with pytest.raises(ValueError):
        m.sparse_attn_fwd(q, k, v, host)
    with pytest.raises(ValueError):
        m.lpt_order(q, k, host)
    with pytest.raises(ValueError):
        m.to_intervals(host, heads=w.heads)
    vote = m.MaskVote(w.batch, w.heads, w.n_q_blocks, w.n_k_blocks, device="cuda")
    with pytest.raises(ValueError):
        vote.add(host)
    # the same index on the GPU still runs
    m.sparse_attn_fwd(q, k, v, idx)
    vote.add(idx)
    torch.cuda.synchronize()


def test_outputs_on_the_host_are_rejected():
    m = dbsp()
    w = small_variants()["star_mid_small"]
    q, k, v = make_qkv(w, device="cuda", seed=5)
    idx = m.sparse_select(q, k, w.text, w.extra, density=w.param)
    with pytest.raises(ValueError):
        m.sparse_attn_fwd(q, k, v, idx, return_lse=True,
                          lse=torch.empty(q.shape[:3], dtype=torch.float32))
    with pytest.raises(ValueError):  # wrong lse shape
        m.sparse_attn_fwd(q, k, v, idx, return_lse=True,
                          lse=torch.empty(q.shape[:2], dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        m.block_energy(q, k, out=torch.empty((w.rows, w.n_k_blocks), dtype=torch.float32))
    with pytest.raises(ValueError):
        m.lpt_order(q, k, idx, out=torch.empty(w.rows, dtype=torch.int32))
    torch.cuda.synchronize()


@pytest.mark.parametrize("nkb,nqb", [(37, 300), (1500, 1100), (8191, 64), (8200, 300)])
def test_lpt_order_from_a_given_csr(nkb, nqb):
    # the order depends only on the CSR row lengths, so a synthetic CSR drives both sort paths:
    # buckets in LDS per head (up to 8,191 key blocks: one bucket per thread and a single pass
    # over the rows at 37 x 300; several buckets per thread and several passes over the rows at
    # 1,500 x 1,100 (the 720p final scale under a longest-first order has 1,132 key blocks); the
    # largest LDS bucket array at 8,191) and the global-bucket launches beyond
    import ctypes
    from dynamic_block_sparse_pool_amd import _abi
    lib = _abi.load()
    batch, heads = 2, 3
    rows = batch * heads * nqb
    rng = np.random.default_rng(nkb)
    lens = rng.integers(0, nkb + 1, size=rows)
    lens[rng.random(rows) < 0.2] = nkb                     # some rows keep every block
    lens[rng.random(rows) < 0.1] = 0                       # and some none
    rp = np.zeros(rows + 1, np.int64)
    np.cumsum(lens, out=rp[1:])
    say(f"case synthetic CSR: nkb={nkb} rows={rows} nnz={int(rp[-1])}")
    row_ptr = torch.from_numpy(rp.astype(np.int32)).cuda()
    dims = _abi.Dims(batch, heads, nqb * BLOCK, nkb * BLOCK, 128, _abi.DBSP_BF16)
    need = ctypes.c_uint64()
    assert lib.dbsp_row_order_workspace_bytes(ctypes.byref(dims), ctypes.byref(need)) == 0
    ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device="cuda")
    order = torch.empty(rows, dtype=torch.int32, device="cuda")
    st = lib.dbsp_row_order_lpt(ctypes.c_void_p(row_ptr.data_ptr()), ctypes.byref(dims),
                                int(rp[-1]), ctypes.c_void_p(order.data_ptr()),
                                ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    o = order.cpu().numpy()
    assert np.array_equal(np.sort(o), np.arange(rows))      # a permutation
    head = o // nqb
    assert np.array_equal(head, np.repeat(np.arange(batch * heads), nqb))   # heads in order
    for hh in range(batch * heads):
        assert (np.diff(lens[o[head == hh]]) <= 0).all()    # longest first per head
