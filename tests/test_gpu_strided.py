"""Strided Q / K / V / O views: a [batch, L, heads, head_dim] layout seen head-major, keys and
values shared by all heads (head stride 0), and a strided output.

Each strided call is checked against the oracle on the values it reads, with the parity bars of
the contiguous path: pooled scores, every mask row and CSR entry, every output and lse. The
same values in the contiguous layout must also give bit-identical results (the kernels read the
same numbers in the same order)."""
import numpy as np
import pytest
import torch

from synth import BLOCK, WORKLOADS, make_qkv, small_variants
from tests import parity as P
from tests.test_gpu_parity import full_check_small

pytestmark = pytest.mark.gpu


def dbsp():
    import dynamic_block_sparse_pool_amd as m
    return m


def say(msg):
    print(f"[gpu-strided] {msg}", flush=True)


def bshd_view(t):
    """The same values stored as [batch, L, heads, d], viewed as [batch, heads, L, d]."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def run(q, k, v, w, out=None):
    m = dbsp()
    kw = dict(density=w.param) if w.mode == "topk" else dict(mass=w.param)
    idx = m.sparse_select(q, k, w.text, w.extra, return_scores=True, **kw)
    o, lse = m.sparse_attn_fwd(q, k, v, idx, out_dtype=torch.float32, return_lse=True, out=out)
    torch.cuda.synchronize()
    return idx, o, lse


CASES = {
    "bf16 topk": small_variants()["final_small"],
    "bf16 mass partial": small_variants()["dit_mass_small"].with_(lq=19 * BLOCK - 48,
                                                                  lk=19 * BLOCK - 48),
    "fp32 toy": WORKLOADS["toy"].with_(heads=2, lq=1000, lk=900),
}


def bshd_out(w):
    return torch.empty((w.batch, w.lq, w.heads, w.head_dim), dtype=torch.float32,
                       device="cuda").transpose(1, 2)


@pytest.mark.parametrize("name", list(CASES))
def test_bshd_views_against_oracle(name):
    w = CASES[name]
    say(f"case {name}: B={w.batch} H={w.heads} Lq={w.lq} Lk={w.lk} {w.dtype}")
    q, k, v = make_qkv(w, device="cuda", seed=71)
    qv, kv, vv = bshd_view(q), bshd_view(k), bshd_view(v)
    assert not qv.is_contiguous() and torch.equal(qv, q)
    out_v = bshd_out(w)
    assert not out_v.is_contiguous()
    # the strided selection and attention (strided output too) against the oracle
    idx_s, o_s, l_s = full_check_small(w, inputs=(qv, kv, vv), out=out_v)
    assert o_s.data_ptr() == out_v.data_ptr()
    # and bit-identical to the contiguous call on the same values
    idx_c, o_c, l_c = run(q, k, v, w)
    n = idx_c.nnz()
    assert n == idx_s.nnz()
    assert torch.equal(idx_c.row_ptr, idx_s.row_ptr)
    assert torch.equal(idx_c.col_idx[:n], idx_s.col_idx[:n])
    assert torch.equal(idx_c.scores, idx_s.scores)
    assert torch.equal(o_c, o_s) and torch.equal(l_c, l_s)


def test_keys_shared_across_heads_against_oracle():
    # multi-query style: one K and V per batch entry read by every head through a 0 head stride
    w = small_variants()["final_small"].with_(heads=3)
    say("case shared K / V (head stride 0)")
    q, k, v = make_qkv(w, device="cuda", seed=72)
    k1, v1 = k[:, :1].expand(-1, w.heads, -1, -1), v[:, :1].expand(-1, w.heads, -1, -1)
    assert k1.stride(1) == 0
    idx_s, o_s, l_s = full_check_small(w, inputs=(q, k1, v1))
    idx_c, o_c, l_c = run(q, k1.contiguous(), v1.contiguous(), w)
    n = idx_c.nnz()
    assert torch.equal(idx_c.col_idx[:n], idx_s.col_idx[:n])
    assert torch.equal(o_c, o_s) and torch.equal(l_c, l_s)
