"""dbsp_sparse_select_noalloc (selection with its scratch in a static device array) through the C
ABI against dbsp_sparse_select with a caller workspace: the same CSR and the same scores, bit
for bit, on two calls in a row where the second has a smaller input (so stale scratch contents
of the first call cannot leak into the second), in Top-K and in mass mode, and at the full
720p final-scale shape."""
import ctypes

import numpy as np
import pytest
import torch

from synth import WORKLOADS, make_qkv, small_variants

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-noalloc] {msg}", flush=True)


def lib():
    from dynamic_block_sparse_pool_amd import _abi
    return _abi, _abi.load()


def vp(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def select_both(w, seed):
    """Run both entry points on the same inputs; return (with-workspace, no-alloc) results as
    (row_ptr, col_idx[:nnz], scores) host arrays."""
    _abi, L = lib()
    q, k, _ = make_qkv(w, device="cuda", seed=seed)
    dims = _abi.Dims(w.batch, w.heads, w.lq, w.lk, w.head_dim,
                     _abi.DBSP_BF16 if w.dtype == "bf16" else _abi.DBSP_F32)
    mode = _abi.DBSP_TOPK if w.mode == "topk" else _abi.DBSP_MASS
    text, extra = _abi.Range(*w.text), _abi.Range(*w.extra)
    bound = ctypes.c_int64()
    assert L.dbsp_select_nnz_bound(ctypes.byref(dims), mode, w.param, text, extra, -1,
                                   ctypes.byref(bound)) == 0
    need = ctypes.c_uint64()
    assert L.dbsp_select_workspace_bytes(ctypes.byref(dims), mode, ctypes.byref(need)) == 0
    assert need.value <= _abi.DBSP_NOALLOC_SCRATCH_BYTES
    rows, nkb = w.rows, w.n_k_blocks
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for noalloc in (False, True):
        row_ptr = torch.full((rows + 1,), -7, dtype=torch.int32, device="cuda")
        col_idx = torch.full((bound.value,), -7, dtype=torch.int32, device="cuda")
        scores = torch.full((rows, nkb), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            st = L.dbsp_sparse_select_noalloc(vp(q), vp(k), ctypes.byref(dims), text, extra, mode,
                                              w.param, -1, 0.0, vp(row_ptr), vp(col_idx),
                                              bound.value, vp(scores), stream)
        else:
            ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device="cuda")
            st = L.dbsp_sparse_select(vp(q), vp(k), ctypes.byref(dims), text, extra, mode,
                                      w.param, -1, 0.0, vp(row_ptr), vp(col_idx), bound.value,
                                      vp(scores), vp(ws), ws.numel(), stream)
        assert st == 0, f"status {st}"
        torch.cuda.synchronize()
        rp = row_ptr.cpu().numpy()
        out.append((rp, col_idx.cpu().numpy()[:rp[-1]], scores.cpu().numpy()))
    return out


def check_equal(w, seed):
    (rp0, ci0, s0), (rp1, ci1, s1) = select_both(w, seed)
    np.testing.assert_array_equal(rp1, rp0)
    np.testing.assert_array_equal(ci1, ci0)
    np.testing.assert_array_equal(s1, s0)  # bit-identical scores (NaN-free: every slot written)
    assert not np.isnan(s1).any()
    say(f"  {w.name}: nnz {int(rp1[-1])} identical to the workspace call")


@pytest.mark.parametrize("big,small", [("final_small", "star_mid_small"),
                                       ("dit_mass_small", "dit_mass_small")])
def test_noalloc_matches_workspace_call_twice(big, small):
    wb = small_variants()[big]
    ws = small_variants()[small]
    if big == small:  # mass mode: the second call on fewer heads and a shorter sequence
        ws = ws.with_(heads=1, lq=ws.lq - 5 * 128 - 17, lk=ws.lk - 7 * 128 - 17)
    say(f"case {big} then smaller {small}")
    check_equal(wb, seed=31)
    check_equal(ws, seed=32)


def test_noalloc_full_size_then_small():
    w = WORKLOADS["final_720p_clip2"]
    say("case final_720p_clip2 then star_mid_small")
    check_equal(w, seed=0)
    check_equal(small_variants()["star_mid_small"], seed=33)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    _abi, L = lib()
    # 64 heads at the 720p final scale need about 37 MiB of pooled keys
    dims = _abi.Dims(1, 64, 72192, 144896, 128, _abi.DBSP_BF16)
    need = ctypes.c_uint64()
    assert L.dbsp_select_workspace_bytes(ctypes.byref(dims), _abi.DBSP_TOPK,
                                         ctypes.byref(need)) == 0
    assert need.value > _abi.DBSP_NOALLOC_SCRATCH_BYTES
    dummy = ctypes.c_void_p(16)
    st = L.dbsp_sparse_select_noalloc(dummy, dummy, ctypes.byref(dims), _abi.Range(0, 4),
                                      _abi.Range(0, 0), _abi.DBSP_TOPK, 0.09375, -1, 0.0, dummy,
                                      dummy, 1 << 30, None, None)
    assert st == _abi.DBSP_ERR_WORKSPACE
