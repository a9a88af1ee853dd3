"""Host-side checks of libdbsp.so: it loads, exports every function include/dbsp.h declares, and
its argument validation returns the documented status before any GPU work. No call here
reaches a kernel launch, so these run without a GPU."""
import ctypes
import os
import re

import pytest

import oracle
from dynamic_block_sparse_pool_amd import _abi
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dbsp.h")

# Aligned, non-null addresses that are never dereferenced: every call below fails validation
# on the host first.
FAKE = ctypes.c_void_p(1 << 20)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_abi.LIB_PATH):
        from dynamic_block_sparse_pool_amd import build
        build.build()
    return _abi.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dbsp_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree(lib):
    names = declared_functions()
    assert names, "no declarations parsed"
    assert set(names) == set(_abi.SIGNATURES), "binding signatures differ from the header"
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_exports_with_nm(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(dbsp_\w+)", out))
    assert set(declared_functions()) <= exported


def test_version_and_status_strings(lib):
    assert lib.dbsp_version() >= 100
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.dbsp_status_string(code).decode() not in ("", "unknown status")
    assert lib.dbsp_status_string(42).decode() == "unknown status"


def dims_of(w, **kw):
    d = dict(batch=w.batch, heads=w.heads, lq=w.lq, lk=w.lk, head_dim=w.head_dim,
             dtype=_abi.DBSP_F32 if w.dtype == "f32" else _abi.DBSP_BF16)
    d.update(kw)
    return _abi.Dims(**d)


@pytest.mark.parametrize("name", ["toy", "star_mid_clip2", "clip1_early", "final_720p_clip2"])
def test_topk_budget_matches_oracle_reading(lib, name):
    w = WORKLOADS[name]
    dims = dims_of(w)
    out = ctypes.c_int32()
    assert lib.dbsp_topk_budget(ctypes.byref(dims), w.param, _abi.Range(*w.text),
                                _abi.Range(*w.extra), -1, ctypes.byref(out)) == 0
    forced = oracle.forced_blocks(w.n_k_blocks, w.text, w.extra)
    assert out.value == oracle.topk_budget(w.param, int((~forced).sum()))
    nnz = ctypes.c_int64()
    assert lib.dbsp_select_nnz_bound(ctypes.byref(dims), _abi.DBSP_TOPK, w.param,
                                     _abi.Range(*w.text), _abi.Range(*w.extra), -1,
                                     ctypes.byref(nnz)) == 0
    assert nnz.value == w.rows * (int(forced.sum()) + out.value)


def test_budget_edge_cases(lib):
    dims = _abi.Dims(1, 1, 128, 8 * 128, 128, _abi.DBSP_BF16)
    out = ctypes.c_int32()
    r0 = _abi.Range(0, 0)
    assert lib.dbsp_topk_budget(ctypes.byref(dims), 0.0, r0, r0, -1, ctypes.byref(out)) == 0
    assert out.value == 0
    assert lib.dbsp_topk_budget(ctypes.byref(dims), 1.0, r0, r0, -1, ctypes.byref(out)) == 0
    assert out.value == 8
    assert lib.dbsp_topk_budget(ctypes.byref(dims), 0.3, r0, r0, 5, ctypes.byref(out)) == 0
    assert out.value == 5
    for bad_density in (-0.1, 1.5, float("nan")):
        assert lib.dbsp_topk_budget(ctypes.byref(dims), bad_density, r0, r0, -1,
                                    ctypes.byref(out)) == _abi.DBSP_ERR_INVALID_ARG
    assert lib.dbsp_topk_budget(ctypes.byref(dims), 0.5, r0, r0, 9,
                                ctypes.byref(out)) == _abi.DBSP_ERR_INVALID_ARG
    # overlapping, reversed and out-of-range forced ranges
    for t, e in (((0, 3), (2, 4)), ((3, 2), (0, 0)), ((0, 9), (0, 0)), ((-1, 2), (0, 0))):
        assert lib.dbsp_topk_budget(ctypes.byref(dims), 0.5, _abi.Range(*t), _abi.Range(*e), -1,
                                    ctypes.byref(out)) == _abi.DBSP_ERR_INVALID_ARG


def test_mass_bound_and_workspace(lib):
    w = WORKLOADS["dit_mass"]
    dims = dims_of(w)
    nnz = ctypes.c_int64()
    r0 = _abi.Range(0, 0)
    assert lib.dbsp_select_nnz_bound(ctypes.byref(dims), _abi.DBSP_MASS, 0.9, r0, r0, -1,
                                     ctypes.byref(nnz)) == 0
    assert nnz.value == w.rows * w.n_k_blocks
    for bad_tau in (0.0, -0.5, 1.01):
        assert lib.dbsp_select_nnz_bound(ctypes.byref(dims), _abi.DBSP_MASS, bad_tau, r0, r0, -1,
                                         ctypes.byref(nnz)) == _abi.DBSP_ERR_INVALID_ARG
    ws_topk, ws_mass = ctypes.c_uint64(), ctypes.c_uint64()
    assert lib.dbsp_select_workspace_bytes(ctypes.byref(dims), _abi.DBSP_TOPK, ctypes.byref(ws_topk)) == 0
    assert lib.dbsp_select_workspace_bytes(ctypes.byref(dims), _abi.DBSP_MASS, ctypes.byref(ws_mass)) == 0
    # pooled keys (bf16 hi and lo halves, tiles of 16 key blocks); pooled queries stay on chip
    pooled_keys = w.batch * w.heads * (-(-w.n_k_blocks // 16) * 16) * w.head_dim * 4
    assert ws_topk.value >= pooled_keys and ws_mass.value > ws_topk.value


def _select(lib, dims, mode=_abi.DBSP_TOPK, param=0.5, text=(0, 1), extra=(0, 0), q=FAKE, k=FAKE,
            row_ptr=FAKE, col_idx=FAKE, cap=1 << 40, ws=FAKE, ws_bytes=1 << 40, override=-1):
    return lib.dbsp_sparse_select(q, k, ctypes.byref(dims), _abi.Range(*text), _abi.Range(*extra),
                                  mode, param, override, 0.0, row_ptr, col_idx, cap, None, ws,
                                  ws_bytes, None)


def test_select_rejects_bad_arguments(lib):
    good = _abi.Dims(1, 2, 256, 1024, 128, _abi.DBSP_BF16)
    E = _abi
    assert _select(lib, good, q=None) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, good, k=None) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, good, row_ptr=None) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, good, col_idx=None) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, good, q=ctypes.c_void_p((1 << 20) + 2)) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, _abi.Dims(1, 2, 0, 1024, 128, E.DBSP_BF16)) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, _abi.Dims(1, 2, 256, 0, 128, E.DBSP_BF16)) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, _abi.Dims(1, 2, 256, -128, 128, E.DBSP_BF16)) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, _abi.Dims(0, 2, 256, 1024, 128, E.DBSP_BF16)) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, _abi.Dims(1, 2, 256, 1024, 128, 7)) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, _abi.Dims(1, 2, 256, 1024, 96, E.DBSP_BF16)) == E.DBSP_ERR_UNSUPPORTED
    assert _select(lib, _abi.Dims(1, 1, 256, 2049 * 128, 128, E.DBSP_BF16)) == E.DBSP_ERR_UNSUPPORTED
    assert _select(lib, good, mode=5) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, good, param=1.5) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, good, mode=E.DBSP_MASS, param=0.0) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, good, text=(0, 3), extra=(2, 5)) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, good, text=(0, 9)) == E.DBSP_ERR_INVALID_ARG
    assert _select(lib, good, override=8) == E.DBSP_ERR_INVALID_ARG
    # capacity: 2 heads x 2 query blocks x (1 forced + ceil(0.5 * 7) = 4) = 20 entries
    assert _select(lib, good, cap=19) == E.DBSP_ERR_CAPACITY
    assert _select(lib, good, cap=19, mode=E.DBSP_MASS, param=0.9) == E.DBSP_ERR_CAPACITY
    assert _select(lib, good, ws=None) == E.DBSP_ERR_WORKSPACE
    assert _select(lib, good, ws_bytes=16) == E.DBSP_ERR_WORKSPACE
    assert _select(lib, good, ws=ctypes.c_void_p((1 << 20) + 16)) == E.DBSP_ERR_WORKSPACE


def test_attn_rejects_bad_arguments(lib):
    E = _abi
    good = _abi.Dims(1, 2, 256, 1024, 128, E.DBSP_BF16)

    def attn(dims=good, q=FAKE, k=FAKE, v=FAKE, rp=FAKE, ci=FAKE, cap=16, scale=0.0, o=FAKE,
             odt=E.DBSP_F32):
        return lib.dbsp_sparse_attn_fwd(q, k, v, ctypes.byref(dims), rp, ci, cap, scale, o, odt,
                                        None, None)

    for kw in ({"q": None}, {"k": None}, {"v": None}, {"rp": None}, {"o": None}, {"ci": None},
               {"cap": -1}, {"odt": 3}, {"scale": float("inf")},
               {"v": ctypes.c_void_p((1 << 20) + 8)},
               {"dims": _abi.Dims(1, 2, 256, 0, 128, E.DBSP_BF16)}):
        assert attn(**kw) == E.DBSP_ERR_INVALID_ARG, kw
    assert attn(dims=_abi.Dims(1, 2, 256, 1024, 64, E.DBSP_BF16)) == E.DBSP_ERR_UNSUPPORTED
    assert attn(dims=_abi.Dims(1, 2, 256, 1024, 32, E.DBSP_F32)) == E.DBSP_ERR_UNSUPPORTED


def test_energy_calls_reject_bad_arguments(lib):
    E = _abi
    good = _abi.Dims(1, 2, 256, 1024, 128, E.DBSP_BF16)

    def energy(dims=good, q=FAKE, k=FAKE, out=FAKE, lse=None, scale=0.0, ws=FAKE, ws_n=1 << 20):
        return lib.dbsp_block_energy(q, k, ctypes.byref(dims), scale, out, lse, ws, ws_n, None)

    for kw in ({"q": None}, {"k": None}, {"out": None}, {"scale": float("nan")},
               {"q": ctypes.c_void_p((1 << 20) + 8)}, {"out": ctypes.c_void_p((1 << 20) + 2)},
               {"dims": _abi.Dims(1, 2, 0, 1024, 128, E.DBSP_BF16)}):
        assert energy(**kw) == E.DBSP_ERR_INVALID_ARG, kw
    assert energy(dims=_abi.Dims(1, 2, 256, 1024, 64, E.DBSP_BF16)) == E.DBSP_ERR_UNSUPPORTED
    assert energy(dims=_abi.Dims(1, 1, 256, 2049 * 128, 128, E.DBSP_BF16)) == E.DBSP_ERR_UNSUPPORTED
    # bf16 needs at least one workgroup's slot (8 key blocks x 128 queries x 4 bytes), 256-aligned
    for kw in ({"ws": None}, {"ws_n": 8 * 512 - 1}, {"ws": ctypes.c_void_p((1 << 20) + 16)}):
        assert energy(**kw) == E.DBSP_ERR_WORKSPACE, kw

    need = ctypes.c_uint64()
    assert lib.dbsp_block_energy_workspace_bytes(ctypes.byref(good), ctypes.byref(need)) == E.DBSP_OK
    assert need.value == 4 * 8 * 512  # min(rows = 4, 512) slots of 8 blocks x 128 floats
    big = _abi.Dims(1, 40, 75648, 75648, 128, E.DBSP_BF16)  # 23,640 rows: 512 slots
    assert lib.dbsp_block_energy_workspace_bytes(ctypes.byref(big), ctypes.byref(need)) == E.DBSP_OK
    assert need.value == 512 * 591 * 512
    f32 = _abi.Dims(1, 2, 256, 1024, 128, E.DBSP_F32)
    assert lib.dbsp_block_energy_workspace_bytes(ctypes.byref(f32), ctypes.byref(need)) == E.DBSP_OK
    assert need.value == 0
    assert lib.dbsp_block_energy_workspace_bytes(None, ctypes.byref(need)) == E.DBSP_ERR_INVALID_ARG

    def mass(dims=good, e=FAKE, rp=FAKE, ci=FAKE, cap=16, out=FAKE):
        return lib.dbsp_retained_mass(e, ctypes.byref(dims), rp, ci, cap, out, None)

    for kw in ({"e": None}, {"rp": None}, {"out": None}, {"cap": -1}, {"ci": None}):
        assert mass(**kw) == E.DBSP_ERR_INVALID_ARG, kw

    def sel(dims=good, e=FAKE, tau=0.9, text=(0, 1), extra=(0, 0), rp=FAKE, ci=FAKE,
            cap=1 << 40, ws=FAKE, ws_bytes=1 << 40):
        return lib.dbsp_select_energy(e, ctypes.byref(dims), _abi.Range(*text), _abi.Range(*extra),
                                      tau, rp, ci, cap, ws, ws_bytes, None)

    for kw in ({"e": None}, {"rp": None}, {"ci": None}, {"tau": 0.0}, {"tau": 1.5},
               {"text": (0, 9)}, {"text": (0, 3), "extra": (2, 5)}):
        assert sel(**kw) == E.DBSP_ERR_INVALID_ARG, kw
    # 2 heads x 2 query blocks x 8 key blocks
    assert sel(cap=31) == E.DBSP_ERR_CAPACITY
    assert sel(ws=None) == E.DBSP_ERR_WORKSPACE
    assert sel(ws_bytes=16) == E.DBSP_ERR_WORKSPACE
    assert sel(dims=_abi.Dims(1, 1, 256, 2049 * 128, 128, E.DBSP_BF16)) == E.DBSP_ERR_UNSUPPORTED
    ws = ctypes.c_uint64()
    assert lib.dbsp_select_energy_workspace_bytes(ctypes.byref(good), ctypes.byref(ws)) == 0
    rows, words = 4, 1
    assert ws.value >= rows * 4 + rows * words * 8


def test_attn_rejects_too_many_bf16_key_blocks(lib):
    E = _abi
    dims = _abi.Dims(1, 1, 128, 65536 * 128, 128, E.DBSP_BF16)
    assert lib.dbsp_sparse_attn_fwd(FAKE, FAKE, FAKE, ctypes.byref(dims), FAKE, FAKE, 16, 0.0, FAKE,
                                    E.DBSP_F32, None, None) == E.DBSP_ERR_UNSUPPORTED


def test_vote_calls_reject_bad_arguments(lib):
    E = _abi
    good = _abi.Dims(1, 2, 256, 1024, 128, E.DBSP_BF16)

    def acc(dims=good, rp=FAKE, ci=FAKE, cap=16, counts=FAKE):
        return lib.dbsp_vote_accumulate(rp, ci, cap, ctypes.byref(dims), counts, None)

    for kw in ({"rp": None}, {"counts": None}, {"cap": -1}, {"ci": None},
               {"dims": _abi.Dims(1, 2, 256, 0, 128, E.DBSP_BF16)}):
        assert acc(**kw) == E.DBSP_ERR_INVALID_ARG, kw

    def sel(dims=good, counts=FAKE, n=4, rho=0.5, rp=FAKE, ci=FAKE, cap=1 << 40, ws=FAKE,
            ws_bytes=1 << 40):
        return lib.dbsp_vote_select(counts, ctypes.byref(dims), n, rho, rp, ci, cap, ws, ws_bytes,
                                    None)

    for kw in ({"counts": None}, {"rp": None}, {"ci": None}, {"n": 0}, {"rho": -0.1},
               {"rho": 1.5}, {"rho": float("nan")}):
        assert sel(**kw) == E.DBSP_ERR_INVALID_ARG, kw
    assert sel(cap=31) == E.DBSP_ERR_CAPACITY      # 4 rows x 8 key blocks
    assert sel(ws=None) == E.DBSP_ERR_WORKSPACE
    assert sel(ws=ctypes.c_void_p((1 << 20) + 16)) == E.DBSP_ERR_WORKSPACE
    ws = ctypes.c_uint64()
    assert lib.dbsp_vote_workspace_bytes(ctypes.byref(good), ctypes.byref(ws)) == 0 and ws.value > 0


def test_forced_list_validation(lib):
    E = _abi
    dims = _abi.Dims(1, 2, 256, 1024, 128, E.DBSP_BF16)   # 8 key blocks, 4 rows

    def bound(lst, mode=E.DBSP_TOPK, param=0.5):
        arr = (ctypes.c_int32 * max(len(lst), 1))(*lst) if lst else None
        out = ctypes.c_int64()
        st = lib.dbsp_select_nnz_bound_list(ctypes.byref(dims), mode, param, arr, len(lst), -1,
                                            ctypes.byref(out))
        return st, out.value

    # scattered list {1, 6}: |C| = 6, K = ceil(0.5 * 6) = 3 -> 4 rows x 5
    assert bound([6, 1]) == (0, 4 * 5)
    assert bound([]) == (0, 4 * 4)            # no forced block: K = ceil(0.5 * 8)
    assert bound([3], E.DBSP_MASS, 0.9) == (0, 4 * 8)
    for bad in ([8], [-1], [2, 2], [0, 5, 0]):
        assert bound(bad)[0] == E.DBSP_ERR_INVALID_ARG, bad
    # the same checks guard the select call itself, before any workspace check
    arr = (ctypes.c_int32 * 2)(3, 3)
    assert lib.dbsp_sparse_select_list(FAKE, FAKE, ctypes.byref(dims), arr, 2, E.DBSP_TOPK, 0.5,
                                       -1, 0.0, FAKE, FAKE, 1 << 40, None, None, 0,
                                       None) == E.DBSP_ERR_INVALID_ARG
    assert lib.dbsp_sparse_select_list(FAKE, FAKE, ctypes.byref(dims), None, 1, E.DBSP_TOPK, 0.5,
                                       -1, 0.0, FAKE, FAKE, 1 << 40, None, None, 0,
                                       None) == E.DBSP_ERR_INVALID_ARG
    ok = (ctypes.c_int32 * 2)(1, 6)
    assert lib.dbsp_sparse_select_list(FAKE, FAKE, ctypes.byref(dims), ok, 2, E.DBSP_TOPK, 0.5,
                                       -1, 0.0, FAKE, FAKE, 1 << 40, None, None, 0,
                                       None) == E.DBSP_ERR_WORKSPACE


def test_partial_block_shapes_are_counted_by_ceil(lib):
    # lengths that are not multiples of 128 end in a partial block: lk = 1000 -> 8 key blocks,
    # lq = 200 -> 2 query blocks per head
    dims = _abi.Dims(1, 2, 200, 1000, 128, _abi.DBSP_BF16)
    k = ctypes.c_int32()
    assert lib.dbsp_topk_budget(ctypes.byref(dims), 0.5, _abi.Range(0, 1), _abi.Range(0, 0), -1,
                                ctypes.byref(k)) == 0
    assert k.value == 4                                   # ceil(0.5 * 7)
    nnz = ctypes.c_int64()
    assert lib.dbsp_select_nnz_bound(ctypes.byref(dims), _abi.DBSP_MASS, 0.9, _abi.Range(0, 1),
                                     _abi.Range(0, 0), -1, ctypes.byref(nnz)) == 0
    assert nnz.value == 2 * 2 * 8
    ws = ctypes.c_uint64()
    assert lib.dbsp_select_energy_workspace_bytes(ctypes.byref(dims), ctypes.byref(ws)) == 0


def test_skiplist_calls_reject_bad_arguments(lib):
    E = _abi
    dims = _abi.Dims(1, 2, 256, 1000, 128, E.DBSP_BF16)   # 4 rows, 8 key blocks

    def enc(rp=FAKE, ci=FAKE, cap=16, ivp=FAKE, iv=FAKE, ivcap=16, ws=FAKE, wsb=1 << 20):
        return lib.dbsp_csr_to_intervals(rp, ci, cap, ctypes.byref(dims), ivp, iv, ivcap, ws, wsb,
                                         None)

    for kw in ({"rp": None}, {"ivp": None}, {"iv": None}, {"ci": None}, {"cap": -1},
               {"ivcap": -1}):
        assert enc(**kw) == E.DBSP_ERR_INVALID_ARG, kw
    assert enc(ivcap=15) == E.DBSP_ERR_CAPACITY          # 4 rows x ceil(8 / 2) runs
    assert enc(ws=None) == E.DBSP_ERR_WORKSPACE
    assert enc(wsb=8) == E.DBSP_ERR_WORKSPACE

    def dec(ivp=FAKE, iv=FAKE, ivcap=16, rp=FAKE, ci=FAKE, cap=32, ws=FAKE, wsb=1 << 20):
        return lib.dbsp_intervals_to_csr(ivp, iv, ivcap, ctypes.byref(dims), rp, ci, cap, ws, wsb,
                                         None)

    for kw in ({"ivp": None}, {"rp": None}, {"ci": None}, {"iv": None}, {"ivcap": -1},
               {"cap": -1}):
        assert dec(**kw) == E.DBSP_ERR_INVALID_ARG, kw
    assert dec(cap=31) == E.DBSP_ERR_CAPACITY             # 4 rows x 8 blocks
    assert dec(ws=ctypes.c_void_p((1 << 20) + 8)) == E.DBSP_ERR_WORKSPACE


def test_strided_calls_reject_bad_strides(lib):
    E = _abi
    dims = _abi.Dims(1, 2, 256, 1024, 128, E.DBSP_BF16)
    good = _abi.Strides(2 * 256 * 128, 256 * 128, 128)

    def attn(qs=good, ks=good, vs=good, os_=_abi.Strides(2 * 256 * 128, 256 * 128, 128),
             odt=E.DBSP_F32):
        args = [ctypes.byref(x) if x is not None else None for x in (qs, ks, vs, os_)]
        return lib.dbsp_sparse_attn_fwd_strided(FAKE, args[0], FAKE, args[1], FAKE, args[2],
                                                ctypes.byref(dims), FAKE, FAKE, 16, 0.0, FAKE,
                                                args[3], odt, None, None)

    for kw in ({"qs": None}, {"os_": None},
               {"ks": _abi.Strides(-1, 128, 128)},              # negative
               {"qs": _abi.Strides(0, 0, 100)},                 # rows not 16-byte aligned
               {"os_": _abi.Strides(0, 0, 64)}):                # output rows overlap
        assert attn(**kw) == E.DBSP_ERR_INVALID_ARG, kw

    def sel(qs=good, ks=good):
        args = [ctypes.byref(x) if x is not None else None for x in (qs, ks)]
        return lib.dbsp_sparse_select_strided(FAKE, args[0], FAKE, args[1], ctypes.byref(dims),
                                              _abi.Range(0, 1), _abi.Range(0, 0), E.DBSP_TOPK,
                                              0.5, -1, 0.0, FAKE, FAKE, 1 << 40, None, None, 0,
                                              None)

    assert sel(ks=None) == E.DBSP_ERR_INVALID_ARG
    assert sel(qs=_abi.Strides(0, 3, 128)) == E.DBSP_ERR_INVALID_ARG
    assert sel() == E.DBSP_ERR_WORKSPACE      # valid strides reach the workspace check


def test_row_order_calls_reject_bad_arguments(lib):
    E = _abi
    dims = _abi.Dims(1, 2, 256, 1000, 128, E.DBSP_BF16)   # 4 rows, 8 key blocks
    need = ctypes.c_uint64(0)
    assert lib.dbsp_row_order_workspace_bytes(ctypes.byref(dims), ctypes.byref(need)) == E.DBSP_OK
    assert need.value == 256 + 4 * (2 * 9 + 1)  # counts (aligned) + cursors, 2 heads x 9 buckets
    assert lib.dbsp_row_order_workspace_bytes(None, ctypes.byref(need)) == E.DBSP_ERR_INVALID_ARG
    assert lib.dbsp_row_order_workspace_bytes(ctypes.byref(dims), None) == E.DBSP_ERR_INVALID_ARG

    def order(rp=FAKE, cap=16, out=FAKE, ws=FAKE, wsb=1 << 20):
        return lib.dbsp_row_order_lpt(rp, ctypes.byref(dims), cap, out, ws, wsb, None)

    for kw in ({"rp": None}, {"out": None}, {"cap": -1}):
        assert order(**kw) == E.DBSP_ERR_INVALID_ARG, kw
    assert order(ws=None) == E.DBSP_ERR_WORKSPACE
    assert order(wsb=need.value - 1) == E.DBSP_ERR_WORKSPACE
    assert order(ws=ctypes.c_void_p((1 << 20) + 64)) == E.DBSP_ERR_WORKSPACE  # not 256-aligned

    def attn(row_order=FAKE, rp=FAKE):
        return lib.dbsp_sparse_attn_fwd_ordered(FAKE, FAKE, FAKE, ctypes.byref(dims), rp, FAKE, 16,
                                                0.0, FAKE, E.DBSP_F32, None, row_order, None)

    assert attn(row_order=None) == E.DBSP_ERR_INVALID_ARG
    assert attn(rp=None) == E.DBSP_ERR_INVALID_ARG


def test_noalloc_select_rejects_before_gpu_work(lib):
    # the size check of the static scratch and the argument checks run on the host first
    w = WORKLOADS["final_720p_clip2"]
    big = dims_of(w, heads=64)              # ~37 MiB of pooled keys > the 32 MiB scratch
    need = ctypes.c_uint64()
    assert lib.dbsp_select_workspace_bytes(ctypes.byref(big), _abi.DBSP_TOPK,
                                           ctypes.byref(need)) == 0
    assert need.value > _abi.DBSP_NOALLOC_SCRATCH_BYTES
    args = (_abi.Range(0, 4), _abi.Range(0, 0), _abi.DBSP_TOPK, 0.09375, -1, 0.0, FAKE, FAKE,
            1 << 30, None, None)
    assert lib.dbsp_sparse_select_noalloc(FAKE, FAKE, ctypes.byref(big), *args) == \
        _abi.DBSP_ERR_WORKSPACE
    assert lib.dbsp_sparse_select_noalloc(FAKE, FAKE, None, *args) == _abi.DBSP_ERR_INVALID_ARG
    bad_mode = (args[0], args[1], 7) + args[3:]
    assert lib.dbsp_sparse_select_noalloc(FAKE, FAKE, ctypes.byref(dims_of(w)), *bad_mode) == \
        _abi.DBSP_ERR_INVALID_ARG
