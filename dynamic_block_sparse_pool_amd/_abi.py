"""ctypes declarations for libdbsp.so (include/dbsp.h). Loading fails loudly when the library
is missing: there is no fallback implementation."""
from __future__ import annotations

import ctypes
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libdbsp.so")

DBSP_BLOCK = 128
DBSP_MAX_KEY_BLOCKS = 2048
DBSP_NOALLOC_SCRATCH_BYTES = 32 << 20

DBSP_OK = 0
DBSP_ERR_INVALID_ARG = -1
DBSP_ERR_UNSUPPORTED = -2
DBSP_ERR_CAPACITY = -3
DBSP_ERR_WORKSPACE = -4
DBSP_ERR_HIP = -5

DBSP_F32 = 0
DBSP_BF16 = 1
DBSP_TOPK = 0
DBSP_MASS = 1


class Range(ctypes.Structure):
    _fields_ = [("begin", ctypes.c_int32), ("end", ctypes.c_int32)]


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("lq", ctypes.c_int32),
                ("lk", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("token", ctypes.c_int64)]


_i32, _i64, _u64, _f32, _f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_double
_vp = ctypes.c_void_p
_PDims = ctypes.POINTER(Dims)
_PStr = ctypes.POINTER(Strides)

# name -> (restype, argtypes); the order of arguments follows include/dbsp.h
SIGNATURES = {
    "dbsp_version": (_i32, []),
    "dbsp_status_string": (ctypes.c_char_p, [_i32]),
    "dbsp_topk_budget": (_i32, [_PDims, _f64, Range, Range, _i32, ctypes.POINTER(_i32)]),
    "dbsp_select_nnz_bound": (_i32, [_PDims, _i32, _f64, Range, Range, _i32, ctypes.POINTER(_i64)]),
    "dbsp_select_workspace_bytes": (_i32, [_PDims, _i32, ctypes.POINTER(_u64)]),
    "dbsp_sparse_select": (_i32, [_vp, _vp, _PDims, Range, Range, _i32, _f64, _i32, _f32,
                                  _vp, _vp, _i64, _vp, _vp, _u64, _vp]),
    "dbsp_sparse_attn_fwd": (_i32, [_vp, _vp, _vp, _PDims, _vp, _vp, _i64, _f32, _vp, _i32, _vp,
                                    _vp]),
    "dbsp_sparse_select_noalloc": (_i32, [_vp, _vp, _PDims, Range, Range, _i32, _f64, _i32, _f32,
                                          _vp, _vp, _i64, _vp, _vp]),
    "dbsp_sparse_select_strided": (_i32, [_vp, _PStr, _vp, _PStr, _PDims, Range, Range, _i32,
                                          _f64, _i32, _f32, _vp, _vp, _i64, _vp, _vp, _u64,
                                          _vp]),
    "dbsp_sparse_attn_fwd_strided": (_i32, [_vp, _PStr, _vp, _PStr, _vp, _PStr, _PDims, _vp, _vp,
                                            _i64, _f32, _vp, _PStr, _i32, _vp, _vp]),
    "dbsp_sparse_attn_fwd_ordered": (_i32, [_vp, _vp, _vp, _PDims, _vp, _vp, _i64, _f32, _vp,
                                            _i32, _vp, _vp, _vp]),
    "dbsp_row_order_workspace_bytes": (_i32, [_PDims, ctypes.POINTER(_u64)]),
    "dbsp_row_order_lpt": (_i32, [_vp, _PDims, _i64, _vp, _vp, _u64, _vp]),
    "dbsp_sparse_select_list": (_i32, [_vp, _vp, _PDims, _vp, _i32, _i32, _f64, _i32, _f32,
                                       _vp, _vp, _i64, _vp, _vp, _u64, _vp]),
    "dbsp_select_nnz_bound_list": (_i32, [_PDims, _i32, _f64, _vp, _i32, _i32,
                                          ctypes.POINTER(_i64)]),
    "dbsp_block_energy_workspace_bytes": (_i32, [_PDims, ctypes.POINTER(_u64)]),
    "dbsp_block_energy": (_i32, [_vp, _vp, _PDims, _f32, _vp, _vp, _vp, _u64, _vp]),
    "dbsp_retained_mass": (_i32, [_vp, _PDims, _vp, _vp, _i64, _vp, _vp]),
    "dbsp_select_energy": (_i32, [_vp, _PDims, Range, Range, _f64, _vp, _vp, _i64, _vp, _u64,
                                  _vp]),
    "dbsp_select_energy_workspace_bytes": (_i32, [_PDims, ctypes.POINTER(_u64)]),
    "dbsp_vote_accumulate": (_i32, [_vp, _vp, _i64, _PDims, _vp, _vp]),
    "dbsp_vote_workspace_bytes": (_i32, [_PDims, ctypes.POINTER(_u64)]),
    "dbsp_vote_select": (_i32, [_vp, _PDims, _i32, _f64, _vp, _vp, _i64, _vp, _u64, _vp]),
    "dbsp_skiplist_workspace_bytes": (_i32, [_PDims, ctypes.POINTER(_u64)]),
    "dbsp_csr_to_intervals": (_i32, [_vp, _vp, _i64, _PDims, _vp, _vp, _i64, _vp, _u64, _vp]),
    "dbsp_intervals_to_csr": (_i32, [_vp, _vp, _i64, _PDims, _vp, _vp, _i64, _vp, _u64, _vp]),
    "dbsp_anchor_workspace_bytes": (_i32, [_PDims, _i32, _i32, _i32, _i32, _i32,
                                           ctypes.POINTER(_u64)]),
    "dbsp_anchor_attn_fwd": (_i32, [_vp, _vp, _vp, _PDims, _i32, _i32, _i32, _i32, _f32, _vp,
                                    _i32, _vp, _vp, _u64, _vp]),
}

_lib = None
_lock = threading.Lock()


class DbspError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load(path: str = LIB_PATH):
    """Load libdbsp.so once and declare its functions. Raises ImportError if it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it with `python -m dynamic_block_sparse_pool_amd.build` "
                "(the HIP library is required; there is no fallback)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().dbsp_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != DBSP_OK:
        raise DbspError(status, where)
