"""Per-head dynamic block-sparse attention for MI355X (gfx950).

Python binding over the C ABI of libdbsp.so (include/dbsp.h). Only argument marshalling
happens here: torch tensors supply device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.

    import dynamic_block_sparse_pool_amd as dbsp
    idx = dbsp.sparse_select(q, k, text_blocks=(0, 4), density=0.09375)
    o = dbsp.sparse_attn_fwd(q, k, v, idx)

q is [batch, heads, Lq, d] and k, v are [batch, heads, Lk, d], contiguous CUDA tensors
(bfloat16 with d = 128, or float32 with d = 64 / 128), Lq and Lk multiples of 128.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional, Tuple

import torch

from . import _abi
from ._abi import DBSP_BLOCK, DbspError

__all__ = ["BlockIndex", "sparse_select", "sparse_attn_fwd", "lpt_order", "topk_budget",
           "select_nnz_bound", "select_workspace_bytes", "block_energy", "block_energy_workspace_bytes", "retained_mass", "select_energy",
           "MaskVote", "anchor_attn_fwd", "to_intervals", "from_intervals",
           "DbspError", "DBSP_BLOCK", "version"]


@dataclasses.dataclass
class BlockIndex:
    """Forward-only CSR skip list: row r = (b * heads + h) * n_q_blocks + i lists the key blocks
    query block i of head h attends to, ascending. nnz lives in row_ptr[-1] on the device."""
    row_ptr: torch.Tensor          # int32 [rows + 1]
    col_idx: torch.Tensor          # int32 [capacity]
    n_q_blocks: int
    n_k_blocks: int
    scores: Optional[torch.Tensor] = None   # float32 [rows, n_k_blocks] if requested

    @property
    def rows(self) -> int:
        return self.row_ptr.numel() - 1

    def nnz(self) -> int:
        """Number of kept (row, key block) pairs; synchronises with the device."""
        return int(self.row_ptr[-1].item())


def _nblocks(length: int) -> int:
    """Blocks of a sequence: a length that is not a multiple of 128 ends in a partial block."""
    return -(-int(length) // DBSP_BLOCK)


def version() -> int:
    return int(_abi.load().dbsp_version())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _abi.DBSP_BF16
    if t.dtype == torch.float32:
        return _abi.DBSP_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _dims(q: torch.Tensor, k: torch.Tensor) -> _abi.Dims:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [batch, heads, L, head_dim]")
    if q.shape[0] != k.shape[0] or q.shape[1] != k.shape[1] or q.shape[3] != k.shape[3]:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} vs k {tuple(k.shape)}")
    if q.dtype != k.dtype:
        raise TypeError("q and k must share a dtype")
    if q.device != k.device:
        raise ValueError("q and k must be on one device")
    return _abi.Dims(q.shape[0], q.shape[1], q.shape[2], k.shape[2], q.shape[3], _dtype_code(q))


def _range(r) -> _abi.Range:
    if r is None:
        return _abi.Range(0, 0)
    b, e = r
    return _abi.Range(int(b), int(e))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_device_tensor(name: str, t: torch.Tensor) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_index(index: "BlockIndex", device: torch.device) -> None:
    """row_ptr and col_idx: contiguous int32 tensors on `device` (the kernels read them)."""
    for name, t in (("row_ptr", index.row_ptr), ("col_idx", index.col_idx)):
        if t.device.type != device.type or (device.index is not None and
                                            t.device.index != device.index):
            raise ValueError(f"index.{name} must be on {device} (it is on {t.device})")
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"index.{name} must be a contiguous int32 tensor")


def _check_on(name: str, t: torch.Tensor, device: torch.device) -> None:
    """A caller-supplied output or workspace must live on the inputs' GPU."""
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (it is on {t.device})")


def _check_view(name: str, t: torch.Tensor) -> None:
    """A 4-D GPU view whose last dimension is contiguous (other strides are passed through)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{name} must be a [batch, heads, L, head_dim] view with contiguous "
                         "head_dim")


def _strides(t: torch.Tensor):
    """None for a contiguous tensor, else its [batch, heads, L] element strides."""
    if t.is_contiguous():
        return None
    return _abi.Strides(t.stride(0), t.stride(1), t.stride(2))


def topk_budget(n_k_blocks: int, density: float, text_blocks=(0, 0), dense_extra_blocks=(0, 0),
                topk_override: int = -1) -> int:
    """K, the number of non-forced key blocks Top-K keeps per row (host-only query)."""
    dims = _abi.Dims(1, 1, DBSP_BLOCK, int(n_k_blocks) * DBSP_BLOCK, 128, _abi.DBSP_BF16)
    out = ctypes.c_int32()
    _abi.check(_abi.load().dbsp_topk_budget(ctypes.byref(dims), float(density), _range(text_blocks),
                                            _range(dense_extra_blocks), int(topk_override),
                                            ctypes.byref(out)), "dbsp_topk_budget")
    return out.value


def select_nnz_bound(dims: _abi.Dims, mode: int, param: float, text_blocks, extra_blocks,
                     topk_override: int = -1) -> int:
    out = ctypes.c_int64()
    _abi.check(_abi.load().dbsp_select_nnz_bound(ctypes.byref(dims), int(mode), float(param),
                                                 _range(text_blocks), _range(extra_blocks),
                                                 int(topk_override), ctypes.byref(out)),
               "dbsp_select_nnz_bound")
    return out.value


def select_workspace_bytes(dims: _abi.Dims, mode: int) -> int:
    out = ctypes.c_uint64()
    _abi.check(_abi.load().dbsp_select_workspace_bytes(ctypes.byref(dims), int(mode),
                                                       ctypes.byref(out)),
               "dbsp_select_workspace_bytes")
    return out.value


class SelectPlan:
    """Buffers for repeated dbsp_sparse_select calls of one shape (CSR, workspace, scores).
    Allocating them once keeps the hot loop free of allocations."""

    def __init__(self, q: torch.Tensor, k: torch.Tensor, text_blocks=(0, 0),
                 dense_extra_blocks=(0, 0), density: Optional[float] = None,
                 mass: Optional[float] = None, topk_override: int = -1,
                 score_scale: float = 0.0, return_scores: bool = False,
                 forced_blocks=None):
        if (density is None) == (mass is None):
            raise ValueError("give exactly one of density (Top-K) or mass (cumulative mass)")
        # an explicit forced list replaces the two ranges
        self.forced = (None if forced_blocks is None else
                       (ctypes.c_int32 * len(forced_blocks))(*[int(c) for c in forced_blocks]))
        _check_view("q", q)
        _check_view("k", k)
        self.dims = _dims(q, k)
        self.mode = _abi.DBSP_TOPK if density is not None else _abi.DBSP_MASS
        self.param = float(density if density is not None else mass)
        self.text = _range(text_blocks)
        self.extra = _range(dense_extra_blocks)
        self.topk_override = int(topk_override)
        self.score_scale = float(score_scale)
        self.device = q.device
        rows = self.dims.batch * self.dims.heads * (_nblocks(self.dims.lq))
        nkb = _nblocks(self.dims.lk)
        if self.forced is None:
            self.capacity = select_nnz_bound(self.dims, self.mode, self.param, text_blocks,
                                             dense_extra_blocks, self.topk_override)
        else:
            out = ctypes.c_int64()
            _abi.check(_abi.load().dbsp_select_nnz_bound_list(
                ctypes.byref(self.dims), self.mode, self.param, self.forced, len(self.forced),
                self.topk_override, ctypes.byref(out)), "dbsp_select_nnz_bound_list")
            self.capacity = out.value
        ws = select_workspace_bytes(self.dims, self.mode)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=q.device)
        self.row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=q.device)
        self.col_idx = torch.empty(max(self.capacity, 1), dtype=torch.int32, device=q.device)
        self.scores = (torch.empty((rows, nkb), dtype=torch.float32, device=q.device)
                       if return_scores else None)
        self.index = BlockIndex(self.row_ptr, self.col_idx, _nblocks(self.dims.lq), nkb,
                                self.scores)

    def run(self, q: torch.Tensor, k: torch.Tensor) -> BlockIndex:
        d = _dims(q, k)
        if (d.batch, d.heads, d.lq, d.lk, d.head_dim, d.dtype) != (
                self.dims.batch, self.dims.heads, self.dims.lq, self.dims.lk, self.dims.head_dim,
                self.dims.dtype):
            raise ValueError("q / k shape or dtype differs from the plan")
        _check_view("q", q)
        _check_view("k", k)
        qs, ks = _strides(q), _strides(k)
        if (qs is not None or ks is not None) and self.forced is not None:
            raise ValueError("strided q / k with a forced list is not supported; pass ranges")
        if qs is not None or ks is not None:
            qs = qs or _abi.Strides(q.stride(0), q.stride(1), q.stride(2))
            ks = ks or _abi.Strides(k.stride(0), k.stride(1), k.stride(2))
            st = _abi.load().dbsp_sparse_select_strided(
                _ptr(q), ctypes.byref(qs), _ptr(k), ctypes.byref(ks), ctypes.byref(self.dims),
                self.text, self.extra, self.mode, self.param, self.topk_override,
                self.score_scale, _ptr(self.row_ptr), _ptr(self.col_idx), self.col_idx.numel(),
                _ptr(self.scores), _ptr(self.workspace), self.workspace.numel(),
                _stream(q.device))
        elif self.forced is None:
            st = _abi.load().dbsp_sparse_select(
                _ptr(q), _ptr(k), ctypes.byref(self.dims), self.text, self.extra, self.mode,
                self.param, self.topk_override, self.score_scale, _ptr(self.row_ptr),
                _ptr(self.col_idx), self.col_idx.numel(), _ptr(self.scores),
                _ptr(self.workspace), self.workspace.numel(), _stream(q.device))
        else:
            st = _abi.load().dbsp_sparse_select_list(
                _ptr(q), _ptr(k), ctypes.byref(self.dims), self.forced, len(self.forced),
                self.mode, self.param, self.topk_override, self.score_scale, _ptr(self.row_ptr),
                _ptr(self.col_idx), self.col_idx.numel(), _ptr(self.scores),
                _ptr(self.workspace), self.workspace.numel(), _stream(q.device))
        _abi.check(st, "dbsp_sparse_select")
        return self.index


def sparse_select(q: torch.Tensor, k: torch.Tensor, text_blocks: Tuple[int, int] = (0, 0),
                  dense_extra_blocks: Tuple[int, int] = (0, 0), density: Optional[float] = None,
                  mass: Optional[float] = None, topk_override: int = -1, score_scale: float = 0.0,
                  return_scores: bool = False, forced_blocks=None) -> BlockIndex:
    """Pool Q and K per 128-token block, score block pairs per head, keep the forced ranges (or
    the explicit `forced_blocks` list, which replaces them) and pick the remaining key blocks per
    (head, query block): Top-K at `density`, or the shortest cumulative-mass prefix reaching
    `mass`. Returns the CSR skip list."""
    plan = SelectPlan(q, k, text_blocks, dense_extra_blocks, density, mass, topk_override,
                      score_scale, return_scores, forced_blocks)
    return plan.run(q, k)


def lpt_order(q: torch.Tensor, k: torch.Tensor, index: BlockIndex,
              out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows of `index` in (batch, head) order, each head's rows sorted by kept count, longest
    first (equal counts in an unspecified order): the row order for
    sparse_attn_fwd(..., row_order=...). int32 [rows]."""
    dims = _dims(q, k)
    if index.row_ptr.numel() != dims.batch * dims.heads * _nblocks(dims.lq) + 1:
        raise ValueError("index was built for a different shape")
    _check_index(index, q.device)
    if out is None:
        out = torch.empty(index.rows, dtype=torch.int32, device=q.device)
    elif out.shape != (index.rows,) or out.dtype != torch.int32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 [rows] tensor")
    need = ctypes.c_uint64(0)
    _abi.check(_abi.load().dbsp_row_order_workspace_bytes(ctypes.byref(dims), ctypes.byref(need)),
               "dbsp_row_order_workspace_bytes")
    if workspace is None or workspace.numel() * workspace.element_size() < need.value:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    _check_on("out", out, q.device)
    _check_on("workspace", workspace, q.device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    st = _abi.load().dbsp_row_order_lpt(_ptr(index.row_ptr), ctypes.byref(dims),
                                        index.col_idx.numel(), _ptr(out), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(q.device))
    _abi.check(st, "dbsp_row_order_lpt")
    return out


def sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, index: BlockIndex,
                    softmax_scale: float = 0.0, out_dtype: Optional[torch.dtype] = None,
                    return_lse: bool = False, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None,
                    row_order: Optional[torch.Tensor] = None):
    """Forward attention of every query block over the tokens of its kept key blocks only.
    Returns O (and lse if return_lse). row_order (int32 [rows], e.g. from lpt_order) sets the
    order in which rows are started; it does not change the result."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_view(name, t)
    dims = _dims(q, k)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    rows = dims.batch * dims.heads * (_nblocks(dims.lq))
    if index.row_ptr.numel() != rows + 1:
        raise ValueError("index was built for a different shape")
    if index.row_ptr.dtype != torch.int32 or index.col_idx.dtype != torch.int32:
        raise TypeError("row_ptr and col_idx must be int32")
    _check_index(index, q.device)
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    odt = out_dtype or (torch.float32 if q.dtype == torch.float32 else torch.bfloat16)
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    elif out.shape != q.shape or out.dtype != odt:
        raise ValueError("out has the wrong shape or dtype")
    _check_view("out", out)
    _check_on("out", out, q.device)
    if return_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != q.shape[:3] or lse.dtype != torch.float32 or
                              not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [batch, heads, Lq] tensor")
    if lse is not None:
        _check_on("lse", lse, q.device)
    if row_order is not None:
        if not all(t.is_contiguous() for t in (q, k, v, out)):
            raise ValueError("row_order needs contiguous q, k, v and out")
        if row_order.shape != (rows,) or row_order.dtype != torch.int32 or \
                not row_order.is_contiguous() or row_order.device != q.device:
            raise ValueError("row_order must be a contiguous int32 [rows] tensor on q's device")
        st = _abi.load().dbsp_sparse_attn_fwd_ordered(
            _ptr(q), _ptr(k), _ptr(v), ctypes.byref(dims), _ptr(index.row_ptr),
            _ptr(index.col_idx), index.col_idx.numel(), float(softmax_scale), _ptr(out),
            _dtype_code(out), _ptr(lse), _ptr(row_order), _stream(q.device))
    elif all(t.is_contiguous() for t in (q, k, v, out)):
        st = _abi.load().dbsp_sparse_attn_fwd(
            _ptr(q), _ptr(k), _ptr(v), ctypes.byref(dims), _ptr(index.row_ptr),
            _ptr(index.col_idx), index.col_idx.numel(), float(softmax_scale), _ptr(out),
            _dtype_code(out), _ptr(lse), _stream(q.device))
    else:
        ss = [_abi.Strides(t.stride(0), t.stride(1), t.stride(2)) for t in (q, k, v, out)]
        st = _abi.load().dbsp_sparse_attn_fwd_strided(
            _ptr(q), ctypes.byref(ss[0]), _ptr(k), ctypes.byref(ss[1]), _ptr(v),
            ctypes.byref(ss[2]), ctypes.byref(dims), _ptr(index.row_ptr), _ptr(index.col_idx),
            index.col_idx.numel(), float(softmax_scale), _ptr(out), ctypes.byref(ss[3]),
            _dtype_code(out), _ptr(lse), _stream(q.device))
    _abi.check(st, "dbsp_sparse_attn_fwd")
    return (out, lse) if return_lse else out


def block_energy_workspace_bytes(q: torch.Tensor, k: torch.Tensor) -> int:
    """Workspace size (bytes) at which block_energy runs with all its workgroups at once (0 for
    float32 inputs)."""
    dims = _dims(q, k)
    need = ctypes.c_uint64()
    _abi.check(_abi.load().dbsp_block_energy_workspace_bytes(ctypes.byref(dims),
                                                             ctypes.byref(need)),
               "dbsp_block_energy_workspace_bytes")
    return need.value


def block_energy(q: torch.Tensor, k: torch.Tensor, softmax_scale: float = 0.0,
                 return_lse: bool = False, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None):
    """Token-level block energy of every (query block, key block) pair of each head: the
    attention probability mass between the two blocks under the dense softmax over all keys,
    divided by 128. Returns a float32 [rows, n_k_blocks] tensor (and the per-query lse).
    `workspace` (uint8, on q's device) is allocated at block_energy_workspace_bytes when None."""
    _check_device_tensor("q", q)
    _check_device_tensor("k", k)
    dims = _dims(q, k)
    rows = dims.batch * dims.heads * (_nblocks(dims.lq))
    nkb = _nblocks(dims.lk)
    if out is None:
        out = torch.empty((rows, nkb), dtype=torch.float32, device=q.device)
    elif out.shape != (rows, nkb) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [rows, n_k_blocks] tensor")
    _check_on("out", out, q.device)
    if workspace is None:
        need = block_energy_workspace_bytes(q, k)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    _check_on("workspace", workspace, q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    st = _abi.load().dbsp_block_energy(_ptr(q), _ptr(k), ctypes.byref(dims), float(softmax_scale),
                                       _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                       _stream(q.device))
    _abi.check(st, "dbsp_block_energy")
    return (out, lse) if return_lse else out


def _energy_dims(energy: torch.Tensor, batch: int, heads: int, n_k_blocks: int) -> _abi.Dims:
    _check_device_tensor("energy", energy)
    if energy.dtype != torch.float32 or energy.dim() != 2 or energy.shape[1] != n_k_blocks:
        raise ValueError("energy must be float32 [rows, n_k_blocks]")
    if energy.shape[0] % (batch * heads):
        raise ValueError("energy rows are not a multiple of batch * heads")
    nqb = energy.shape[0] // (batch * heads)
    # head_dim and dtype do not enter these calls; the values only satisfy the shape check
    return _abi.Dims(batch, heads, nqb * DBSP_BLOCK, n_k_blocks * DBSP_BLOCK, 128, _abi.DBSP_BF16)


def retained_mass(energy: torch.Tensor, index: BlockIndex, batch: int = 1, heads: int = 1):
    """Attention mass each row's mask keeps: the sum of its kept blocks' energies (float64)."""
    dims = _energy_dims(energy, batch, heads, index.n_k_blocks)
    if index.row_ptr.numel() != energy.shape[0] + 1:
        raise ValueError("index and energy have different row counts")
    _check_index(index, energy.device)
    mass = torch.empty(energy.shape[0], dtype=torch.float64, device=energy.device)
    st = _abi.load().dbsp_retained_mass(_ptr(energy), ctypes.byref(dims), _ptr(index.row_ptr),
                                        _ptr(index.col_idx), index.col_idx.numel(), _ptr(mass),
                                        _stream(energy.device))
    _abi.check(st, "dbsp_retained_mass")
    return mass


def select_energy(energy: torch.Tensor, mass: float, text_blocks=(0, 0),
                  dense_extra_blocks=(0, 0), batch: int = 1, heads: int = 1) -> BlockIndex:
    """Cumulative-mass selection on given block probabilities (e.g. token-level energies): per
    row, the forced blocks and then the shortest (energy descending, index ascending) prefix whose
    mass reaches `mass`, returned as an ascending CSR."""
    nkb = energy.shape[1]
    dims = _energy_dims(energy, batch, heads, nkb)
    rows = energy.shape[0]
    cap = select_nnz_bound(dims, _abi.DBSP_MASS, mass, text_blocks, dense_extra_blocks)
    ws_n = ctypes.c_uint64()
    lib = _abi.load()
    _abi.check(lib.dbsp_select_energy_workspace_bytes(ctypes.byref(dims), ctypes.byref(ws_n)),
               "dbsp_select_energy_workspace_bytes")
    ws = torch.empty(max(ws_n.value, 1), dtype=torch.uint8, device=energy.device)
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=energy.device)
    col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=energy.device)
    st = lib.dbsp_select_energy(_ptr(energy), ctypes.byref(dims), _range(text_blocks),
                                _range(dense_extra_blocks), float(mass), _ptr(row_ptr),
                                _ptr(col_idx), col_idx.numel(), _ptr(ws), ws.numel(),
                                _stream(energy.device))
    _abi.check(st, "dbsp_select_energy")
    return BlockIndex(row_ptr, col_idx, _nblocks(dims.lq), nkb, None)


class MaskVote:
    """Cross-input vote of block masks of one shape: add() each calibration input's mask (a
    BlockIndex), then select(rho) keeps the blocks chosen by at least a fraction rho of them
    (exact rational comparison) as one static CSR."""

    def __init__(self, batch: int, heads: int, n_q_blocks: int, n_k_blocks: int,
                 device: torch.device):
        self.dims = _abi.Dims(batch, heads, n_q_blocks * DBSP_BLOCK, n_k_blocks * DBSP_BLOCK, 128,
                              _abi.DBSP_BF16)
        self.rows = batch * heads * n_q_blocks
        self.n_k_blocks = n_k_blocks
        self.n_q_blocks = n_q_blocks
        self.device = torch.device(device)
        self.counts = torch.zeros((self.rows, n_k_blocks), dtype=torch.int32, device=self.device)
        self.n_inputs = 0

    def add(self, index: BlockIndex) -> None:
        if index.row_ptr.numel() != self.rows + 1 or index.n_k_blocks != self.n_k_blocks:
            raise ValueError("mask shape differs from the vote's")
        _check_index(index, self.device)
        st = _abi.load().dbsp_vote_accumulate(_ptr(index.row_ptr), _ptr(index.col_idx),
                                              index.col_idx.numel(), ctypes.byref(self.dims),
                                              _ptr(self.counts), _stream(self.device))
        _abi.check(st, "dbsp_vote_accumulate")
        self.n_inputs += 1

    def select(self, rho: float) -> BlockIndex:
        lib = _abi.load()
        ws_n = ctypes.c_uint64()
        _abi.check(lib.dbsp_vote_workspace_bytes(ctypes.byref(self.dims), ctypes.byref(ws_n)),
                   "dbsp_vote_workspace_bytes")
        ws = torch.empty(max(ws_n.value, 1), dtype=torch.uint8, device=self.device)
        row_ptr = torch.empty(self.rows + 1, dtype=torch.int32, device=self.device)
        col_idx = torch.empty(max(self.rows * self.n_k_blocks, 1), dtype=torch.int32,
                              device=self.device)
        st = lib.dbsp_vote_select(_ptr(self.counts), ctypes.byref(self.dims), self.n_inputs,
                                  float(rho), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                                  _ptr(ws), ws.numel(), _stream(self.device))
        _abi.check(st, "dbsp_vote_select")
        return BlockIndex(row_ptr, col_idx, self.n_q_blocks, self.n_k_blocks, None)


def anchor_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, frames: int,
                    rows_per_frame: int, row_width: int, n_anchors: int = 5,
                    softmax_scale: float = 0.0, out_dtype: Optional[torch.dtype] = None,
                    return_lse: bool = False, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None):
    """Attention of a spatially repeating head: only n_anchors equally spaced rows per frame
    attend (to all keys); every spatial row takes its nearest anchor row's output. Tokens after
    the last frame attend as themselves. Returns O (and lse if return_lse)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_device_tensor(name, t)
    dims = _dims(q, k)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    odt = out_dtype or (torch.float32 if q.dtype == torch.float32 else torch.bfloat16)
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    elif out.shape != q.shape or out.dtype != odt or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    _check_on("out", out, q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    lib = _abi.load()
    n = ctypes.c_uint64()
    geom = (int(frames), int(rows_per_frame), int(row_width), int(n_anchors))
    _abi.check(lib.dbsp_anchor_workspace_bytes(ctypes.byref(dims), *geom, _dtype_code(out),
                                               ctypes.byref(n)), "dbsp_anchor_workspace_bytes")
    if workspace is None or workspace.numel() * workspace.element_size() < n.value:
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=q.device)
    _check_on("workspace", workspace, q.device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    st = lib.dbsp_anchor_attn_fwd(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(dims), *geom,
                                  float(softmax_scale), _ptr(out), _dtype_code(out), _ptr(lse),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(q.device))
    _abi.check(st, "dbsp_anchor_attn_fwd")
    return (out, lse) if return_lse else out


def _skiplist_workspace(dims, device):
    n = ctypes.c_uint64()
    _abi.check(_abi.load().dbsp_skiplist_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)),
               "dbsp_skiplist_workspace_bytes")
    return torch.empty(max(n.value, 1), dtype=torch.uint8, device=device)


def _index_dims(index: BlockIndex, batch: int, heads: int) -> _abi.Dims:
    rows = index.row_ptr.numel() - 1
    if rows % (batch * heads):
        raise ValueError("index rows are not a multiple of batch * heads")
    nqb = rows // (batch * heads)
    return _abi.Dims(batch, heads, nqb * DBSP_BLOCK, index.n_k_blocks * DBSP_BLOCK, 128,
                     _abi.DBSP_BF16)


def to_intervals(index: BlockIndex, batch: int = 1, heads: int = 1):
    """Encode a CSR skip list as maximal runs of key blocks: (iv_ptr [rows + 1] int32, iv
    [capacity, 2] int32 [start, end) pairs; the first iv_ptr[-1] are used)."""
    dims = _index_dims(index, batch, heads)
    dev = index.row_ptr.device
    if not index.row_ptr.is_cuda:
        raise ValueError("index must be on a GPU")
    _check_index(index, dev)
    rows = index.row_ptr.numel() - 1
    cap = rows * ((index.n_k_blocks + 1) // 2)
    iv_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    iv = torch.empty((max(cap, 1), 2), dtype=torch.int32, device=dev)
    ws = _skiplist_workspace(dims, dev)
    st = _abi.load().dbsp_csr_to_intervals(_ptr(index.row_ptr), _ptr(index.col_idx),
                                           index.col_idx.numel(), ctypes.byref(dims),
                                           _ptr(iv_ptr), _ptr(iv), iv.shape[0], _ptr(ws),
                                           ws.numel(), _stream(dev))
    _abi.check(st, "dbsp_csr_to_intervals")
    return iv_ptr, iv


def from_intervals(iv_ptr: torch.Tensor, iv: torch.Tensor, n_q_blocks: int, n_k_blocks: int,
                   batch: int = 1, heads: int = 1) -> BlockIndex:
    """Decode an interval skip list into the CSR the attention call reads."""
    dims = _abi.Dims(batch, heads, n_q_blocks * DBSP_BLOCK, n_k_blocks * DBSP_BLOCK, 128,
                     _abi.DBSP_BF16)
    dev = iv_ptr.device
    rows = batch * heads * n_q_blocks
    if iv_ptr.numel() != rows + 1:
        raise ValueError("iv_ptr has the wrong length")
    _check_device_tensor("iv_ptr", iv_ptr)
    _check_device_tensor("iv", iv)
    _check_on("iv", iv, dev)
    if iv_ptr.dtype != torch.int32 or iv.dtype != torch.int32 or iv.dim() != 2 or iv.shape[1] != 2:
        raise ValueError("iv_ptr must be int32 [rows + 1] and iv int32 [capacity, 2]")
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(rows * n_k_blocks, 1), dtype=torch.int32, device=dev)
    ws = _skiplist_workspace(dims, dev)
    st = _abi.load().dbsp_intervals_to_csr(_ptr(iv_ptr), _ptr(iv), iv.shape[0],
                                           ctypes.byref(dims), _ptr(row_ptr), _ptr(col_idx),
                                           col_idx.numel(), _ptr(ws), ws.numel(), _stream(dev))
    _abi.check(st, "dbsp_intervals_to_csr")
    return BlockIndex(row_ptr, col_idx, n_q_blocks, n_k_blocks, None)
