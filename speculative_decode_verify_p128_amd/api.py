"""PyTorch-facing binding of the verify-attention library.

Argument marshalling only: each function checks that the tensors it is given match the
shapes, dtypes and device the C entry point will address, turns them into pointers,
sizes and a stream handle, and calls the C entry point of the same name; every step of
the path runs in the HIP kernels.  PyTorch supplies device memory and the current
stream.  Output tensors may be passed in (no allocation, e.g. in timed loops) or are
allocated here.

The checks here guard the kernels' addressing: a wrong shape that reached a kernel
would be an out-of-bounds access on the device, so every mismatch is a ValueError or
TypeError before the call.  Row-indexed buffers (q, out, scores, top-k arrays) hold the
capacity of B * max_qo_len rows, as the C header states.

The attention functions take `family` (keyword, default 0): a nonzero family routes the
call to the cross-check build's sdv_xcheck_* entry point, which runs that kernel
implementation on the same arguments (the test suite compares implementations with it).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib as L

_DT = {torch.float32: L.SDV_F32, torch.bfloat16: L.SDV_BF16, torch.float8_e4m3fn: L.SDV_FP8_E4M3}
_OUT_DT = (torch.float32, torch.bfloat16)


def dtype_code(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError(f"unsupported dtype {t}")
    return _DT[t]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, contiguous=True):
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(device, **tensors):
    """`device` is a GPU and every given tensor lives on it (a host tensor's address
    handed to a kernel would be read as device memory)."""
    if device.type != "cuda":
        raise ValueError(f"the call's tensors are on {device}; the library runs on a GPU")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _rows_at_least(t: torch.Tensor, name: str, rows: int, tail: tuple):
    """t is [>= rows, *tail]."""
    if t.dim() != 1 + len(tail) or t.shape[0] < rows or tuple(t.shape[1:]) != tuple(tail):
        raise ValueError(f"{name} must be [>= {rows}, {', '.join(map(str, tail))}], "
                         f"got {tuple(t.shape)}")


def _lengths(qo_indptr: torch.Tensor, kv_len: torch.Tensor) -> int:
    _need(qo_indptr, "qo_indptr", torch.int32)
    _need(kv_len, "kv_len", torch.int32)
    B = kv_len.numel()
    if qo_indptr.numel() != B + 1:
        raise ValueError(f"qo_indptr must hold B + 1 = {B + 1} entries, got {qo_indptr.numel()}")
    return B


def _query(q: torch.Tensor, rows_cap: int, num_kv_heads: int, head_dim: int):
    _need(q, "q")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"q must be float32 or bfloat16, got {q.dtype}")
    if q.dim() != 3:
        raise ValueError(f"q must be [rows, num_q_heads, head_dim], got {tuple(q.shape)}")
    if q.shape[2] != head_dim:
        raise ValueError(f"q head_dim {q.shape[2]} differs from the KV head_dim {head_dim}")
    if q.shape[1] < 1 or q.shape[1] % num_kv_heads != 0:
        raise ValueError(f"num_q_heads {q.shape[1]} is not a multiple of num_kv_heads "
                         f"{num_kv_heads}")
    if q.shape[0] < rows_cap:
        raise ValueError(f"q holds {q.shape[0]} rows, the call addresses B * max_qo_len = "
                         f"{rows_cap}")


def _block_table(bt: torch.Tensor, B: int, name="block_table"):
    _need(bt, name, torch.int32, contiguous=False)
    if bt.dim() != 2 or bt.shape[0] != B or (bt.shape[1] > 0 and bt.stride(1) != 1):
        raise ValueError(f"{name} must be [B = {B}, width] with contiguous rows, got "
                         f"{tuple(bt.shape)} strides {bt.stride()}")


def _dev_err(dev_err):
    if dev_err is not None:
        _need(dev_err, "dev_err", torch.int32)
        if dev_err.numel() < 1:
            raise ValueError("dev_err must hold one int32")


def _call(name: str, family: int, *args) -> None:
    """C entry point `name`, or its cross-check twin for a nonzero kernel family."""
    if family:
        lib = L.load_xcheck()
        L.check(getattr(lib, f"sdv_xcheck_{name}")(family, *args), lib)
    else:
        L.check(getattr(L.load(), name)(*args))


@dataclass
class SubpageView:
    """A validated non-owning P32 view (keeps the pool tensor alive)."""
    c: L.SubpageView
    pool: torch.Tensor

    @property
    def num_kv_heads(self) -> int:
        return self.c.num_kv_heads

    @property
    def head_dim(self) -> int:
        return self.c.head_dim


def kv_subpage_view_init(k_root: torch.Tensor, block_table: torch.Tensor, *, num_kv_heads: int,
                         head_dim: int, slot_stride: int, num_slots: int,
                         k_scale: float = 1.0, v_scale: float = 1.0, pool_index_scale: int = 0,
                         kv_offset: int = 1, num_layers: int = 1, phys_page: int = 128,
                         sub_page: int = 32, max_blocks: Optional[int] = None,
                         sub_offsets: Optional[torch.Tensor] = None,
                         dev_err: Optional[torch.Tensor] = None, stage_offsets: bool = True):
    """k_root: tensor whose first element is slot 0's draft-layer K page.
    block_table: int32 [B, W] P128 slot ids.  Returns (SubpageView, sub_offsets
    int32 [B, 2, 4 * max_blocks]); with stage_offsets=False only the geometry is
    validated (for verify_attention_dense_view) and sub_offsets is None."""
    B = block_table.shape[0] if block_table.dim() == 2 else -1
    _block_table(block_table, B)
    W = block_table.shape[1]
    mb = W if max_blocks is None else max_blocks
    if mb > W:
        raise ValueError(f"max_blocks {mb} exceeds the block table's width {W}")
    dev = block_table.device
    if not stage_offsets:
        B = 0
    elif sub_offsets is None:
        sub_offsets = torch.empty((B, 2, 4 * mb), dtype=torch.int32, device=dev)
    if stage_offsets:
        _need(sub_offsets, "sub_offsets", torch.int32)
        if tuple(sub_offsets.shape) != (B, 2, 4 * mb):
            raise ValueError(f"sub_offsets must be [{B}, 2, {4 * mb}], got {tuple(sub_offsets.shape)}")
    _dev_err(dev_err)
    _same_device(dev, k_root=k_root, sub_offsets=sub_offsets, dev_err=dev_err)
    geom = L.SubpageGeom(phys_page, sub_page, num_kv_heads, head_dim, slot_stride, kv_offset,
                         num_layers, num_slots, pool_index_scale, dtype_code(k_root.dtype),
                         k_scale, v_scale, k_root.data_ptr())
    view = L.SubpageView()
    L.check(L.load().kv_subpage_view_init(C.byref(geom), _ptr(block_table), B, mb,
                                          block_table.stride(0), _ptr(sub_offsets),
                                          C.byref(view), _ptr(dev_err), _stream(dev)))
    return SubpageView(view, k_root), sub_offsets


_OPS = {"dense": L.SDV_OP_VERIFY_DENSE, "sparse": L.SDV_OP_VERIFY_SPARSE,
        "paged": L.SDV_OP_VERIFY_PAGED}


def workspace_bytes(q_rows_cap: int, num_q_heads: int, head_dim: int, num_splits: int,
                    op: str = "dense") -> int:
    """Bytes of split-KV workspace for attention op 'dense', 'sparse' or 'paged'."""
    return int(L.load().sdv_workspace_bytes(_OPS[op], q_rows_cap, num_q_heads, head_dim,
                                            num_splits))


def alloc_workspace(q_rows_cap: int, num_q_heads: int, head_dim: int, num_splits: int, device,
                    op: str = "dense"):
    n = workspace_bytes(q_rows_cap, num_q_heads, head_dim, num_splits, op)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=device)


def _out(out, q, rows_cap, out_dtype):
    if out is None:
        out = torch.empty((rows_cap, q.shape[1], q.shape[2]), dtype=out_dtype or q.dtype,
                          device=q.device)
    _need(out, "out")
    if out.dtype not in _OUT_DT:
        raise TypeError(f"out must be float32 or bfloat16, got {out.dtype}")
    _rows_at_least(out, "out", rows_cap, (q.shape[1], q.shape[2]))
    return out


def _workspace(workspace, rows_cap, q, num_splits, op):
    if workspace is None and num_splits > 1:
        workspace = alloc_workspace(rows_cap, q.shape[1], q.shape[2], num_splits, q.device, op)
    if workspace is not None:
        _need(workspace, "workspace")
    return workspace, 0 if workspace is None else workspace.numel() * workspace.element_size()


def verify_attention_dense(q: torch.Tensor, qo_indptr: torch.Tensor, kv_len: torch.Tensor,
                           view: SubpageView, sub_offsets: torch.Tensor, *, max_qo_len: int,
                           softmax_scale: float, num_splits: int = 1,
                           workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None, out_dtype=None,
                           dev_err: Optional[torch.Tensor] = None, family: int = 0) -> torch.Tensor:
    """q [>= B * max_qo_len, Hq, d]; returns out [B * max_qo_len, Hq, d] (rows of each
    request at qo_indptr[r] ..)."""
    B = _lengths(qo_indptr, kv_len)
    rows_cap = B * max_qo_len
    _query(q, rows_cap, view.num_kv_heads, view.head_dim)
    _need(sub_offsets, "sub_offsets", torch.int32)
    if sub_offsets.dim() != 3 or sub_offsets.shape[0] != B or sub_offsets.shape[1] != 2:
        raise ValueError(f"sub_offsets must be [B = {B}, 2, max_sub_pages], got "
                         f"{tuple(sub_offsets.shape)}")
    out = _out(out, q, rows_cap, out_dtype)
    workspace, ws_bytes = _workspace(workspace, rows_cap, q, num_splits, "dense")
    _dev_err(dev_err)
    _same_device(q.device, qo_indptr=qo_indptr, kv_len=kv_len, sub_offsets=sub_offsets, out=out,
                 workspace=workspace, dev_err=dev_err, pool=view.pool)
    _call("verify_attention_dense", family,
          _ptr(q), dtype_code(q.dtype), _ptr(qo_indptr), _ptr(kv_len), B, max_qo_len, q.shape[1],
          C.byref(view.c), _ptr(sub_offsets), sub_offsets.shape[-1], softmax_scale, num_splits,
          _ptr(workspace), ws_bytes, _ptr(out), dtype_code(out.dtype), _ptr(dev_err),
          _stream(q.device))
    return out


def verify_attention_dense_view(q: torch.Tensor, qo_indptr: torch.Tensor, kv_len: torch.Tensor,
                                view: SubpageView, block_table: torch.Tensor, *, max_qo_len: int,
                                softmax_scale: float, num_splits: int = 1,
                                max_blocks: Optional[int] = None,
                                workspace: Optional[torch.Tensor] = None,
                                out: Optional[torch.Tensor] = None, out_dtype=None,
                                dev_err: Optional[torch.Tensor] = None,
                                family: int = 0) -> torch.Tensor:
    """verify_attention_dense with the view's page indices computed in the attention
    launch from block_table (int32 [B, W] P128 slot ids)."""
    B = _lengths(qo_indptr, kv_len)
    rows_cap = B * max_qo_len
    _query(q, rows_cap, view.num_kv_heads, view.head_dim)
    _block_table(block_table, B)
    mb = block_table.shape[1] if max_blocks is None else max_blocks
    if mb > block_table.shape[1]:
        raise ValueError(f"max_blocks {mb} exceeds the block table's width {block_table.shape[1]}")
    out = _out(out, q, rows_cap, out_dtype)
    workspace, ws_bytes = _workspace(workspace, rows_cap, q, num_splits, "dense")
    _dev_err(dev_err)
    _same_device(q.device, qo_indptr=qo_indptr, kv_len=kv_len, block_table=block_table, out=out,
                 workspace=workspace, dev_err=dev_err, pool=view.pool)
    _call("verify_attention_dense_view", family,
          _ptr(q), dtype_code(q.dtype), _ptr(qo_indptr), _ptr(kv_len), B, max_qo_len, q.shape[1],
          C.byref(view.c), _ptr(block_table), mb, block_table.stride(0), softmax_scale,
          num_splits, _ptr(workspace), ws_bytes, _ptr(out), dtype_code(out.dtype), _ptr(dev_err),
          _stream(q.device))
    return out


def verify_attention_dense_view_noalloc(q: torch.Tensor, qo_indptr: torch.Tensor,
                                        kv_len: torch.Tensor, view: SubpageView,
                                        block_table: torch.Tensor, *, max_qo_len: int,
                                        softmax_scale: float, num_splits: int = 1,
                                        max_blocks: Optional[int] = None,
                                        out: torch.Tensor, dev_err: Optional[torch.Tensor] = None
                                        ) -> torch.Tensor:
    """verify_attention_dense_view with the split-KV partials in the library's device
    scratch (no workspace; `out` must be passed: nothing is allocated)."""
    B = _lengths(qo_indptr, kv_len)
    rows_cap = B * max_qo_len
    _query(q, rows_cap, view.num_kv_heads, view.head_dim)
    _block_table(block_table, B)
    mb = block_table.shape[1] if max_blocks is None else max_blocks
    if mb > block_table.shape[1]:
        raise ValueError(f"max_blocks {mb} exceeds the block table's width {block_table.shape[1]}")
    out = _out(out, q, rows_cap, None)
    _dev_err(dev_err)
    _same_device(q.device, qo_indptr=qo_indptr, kv_len=kv_len, block_table=block_table, out=out,
                 dev_err=dev_err, pool=view.pool)
    L.check(L.load().verify_attention_dense_view_noalloc(
        _ptr(q), dtype_code(q.dtype), _ptr(qo_indptr), _ptr(kv_len), B, max_qo_len, q.shape[1],
        C.byref(view.c), _ptr(block_table), mb, block_table.stride(0), softmax_scale,
        num_splits, _ptr(out), dtype_code(out.dtype), _ptr(dev_err), _stream(q.device)))
    return out


@dataclass
class PagedKV:
    """Head-major P128 page arrays k/v [num_pages, Hkv, 128, d] (non-owning view)."""
    k: torch.Tensor
    v: torch.Tensor
    k_scale: float = 1.0
    v_scale: float = 1.0

    def c(self) -> L.PagedKV:
        if self.k.shape != self.v.shape or self.k.dtype != self.v.dtype:
            raise ValueError("k and v pools must match in shape and dtype")
        if self.k.device != self.v.device:
            raise ValueError("k and v pools must be on one device")
        if not (self.k.is_contiguous() and self.v.is_contiguous()):
            raise ValueError("k and v pools must be contiguous")
        if self.k.dim() != 4:
            raise ValueError(f"k and v pools must be [num_pages, Hkv, 128, d], got "
                             f"{tuple(self.k.shape)}")
        n, H, P, d = self.k.shape
        return L.PagedKV(self.k.data_ptr(), self.v.data_ptr(), H * P * d, n, P, H, d,
                         dtype_code(self.k.dtype), self.k_scale, self.v_scale)


def _scores_shape(scores, rows_cap, Hkv, max_pages):
    _need(scores, "scores", torch.float32)
    _rows_at_least(scores, "scores", rows_cap, (Hkv, max_pages))


def proxy_page_scores(q: torch.Tensor, qo_indptr: torch.Tensor, kv_len: torch.Tensor,
                      kv: PagedKV, block_table: torch.Tensor, *, max_qo_len: int,
                      scores: Optional[torch.Tensor] = None,
                      dev_err: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Returns scores float32 [B * max_qo_len, Hkv, max_pages]."""
    B = _lengths(qo_indptr, kv_len)
    ckv = kv.c()
    rows_cap = B * max_qo_len
    _query(q, rows_cap, ckv.num_kv_heads, ckv.head_dim)
    _block_table(block_table, B)
    max_pages = block_table.shape[1]
    if scores is None:
        scores = torch.empty((rows_cap, ckv.num_kv_heads, max_pages), dtype=torch.float32,
                             device=q.device)
    _scores_shape(scores, rows_cap, ckv.num_kv_heads, max_pages)
    _dev_err(dev_err)
    _same_device(q.device, qo_indptr=qo_indptr, kv_len=kv_len, k=kv.k, block_table=block_table,
                 scores=scores, dev_err=dev_err)
    L.check(L.load().proxy_page_scores(
        _ptr(q), dtype_code(q.dtype), _ptr(qo_indptr), _ptr(kv_len), B, max_qo_len, q.shape[1],
        C.byref(ckv), _ptr(block_table), max_pages, block_table.stride(0), _ptr(scores),
        _ptr(dev_err), _stream(q.device)))
    return scores


def ladder_topk_pages(scores: torch.Tensor, qo_indptr: torch.Tensor, kv_len: torch.Tensor, *,
                      max_qo_len: int, top_k: int, page_size: int = 128,
                      topk_idx: Optional[torch.Tensor] = None,
                      topk_cnt: Optional[torch.Tensor] = None, want_count: bool = False,
                      dev_err: Optional[torch.Tensor] = None):
    """Returns topk_idx int32 [B * max_qo_len, Hkv, top_k] (and counts if asked)."""
    B = _lengths(qo_indptr, kv_len)
    rows_cap = B * max_qo_len
    _need(scores, "scores", torch.float32)
    if scores.dim() != 3:
        raise ValueError(f"scores must be [rows, Hkv, max_pages], got {tuple(scores.shape)}")
    _, Hkv, max_pages = scores.shape
    _scores_shape(scores, rows_cap, Hkv, max_pages)
    if topk_idx is None:
        topk_idx = torch.empty((rows_cap, Hkv, top_k), dtype=torch.int32, device=scores.device)
    if topk_cnt is None and want_count:
        topk_cnt = torch.empty((rows_cap, Hkv), dtype=torch.int32, device=scores.device)
    _topk_shapes(topk_idx, topk_cnt, rows_cap, Hkv, top_k)
    _dev_err(dev_err)
    _same_device(scores.device, qo_indptr=qo_indptr, kv_len=kv_len, topk_idx=topk_idx,
                 topk_cnt=topk_cnt, dev_err=dev_err)
    L.check(L.load().ladder_topk_pages(
        _ptr(scores), _ptr(qo_indptr), _ptr(kv_len), B, max_qo_len, Hkv, max_pages, page_size,
        top_k, _ptr(topk_idx), _ptr(topk_cnt), _ptr(dev_err), _stream(scores.device)))
    return (topk_idx, topk_cnt) if want_count or topk_cnt is not None else topk_idx


def _topk_shapes(topk_idx, topk_cnt, rows_cap, Hkv, top_k):
    if topk_idx is not None:
        _need(topk_idx, "topk_idx", torch.int32)
        _rows_at_least(topk_idx, "topk_idx", rows_cap, (Hkv, top_k))
    if topk_cnt is not None:
        _need(topk_cnt, "topk_cnt", torch.int32)
        _rows_at_least(topk_cnt, "topk_cnt", rows_cap, (Hkv,))


def verify_attention_sparse(q: torch.Tensor, qo_indptr: torch.Tensor, kv_len: torch.Tensor,
                            kv: PagedKV, block_table: torch.Tensor, topk_idx: torch.Tensor, *,
                            max_qo_len: int, softmax_scale: float, num_splits: int = 1,
                            workspace: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None, out_dtype=None,
                            dev_err: Optional[torch.Tensor] = None,
                            family: int = 0) -> torch.Tensor:
    B = _lengths(qo_indptr, kv_len)
    ckv = kv.c()
    rows_cap = B * max_qo_len
    _query(q, rows_cap, ckv.num_kv_heads, ckv.head_dim)
    _block_table(block_table, B)
    _need(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 3:
        raise ValueError(f"topk_idx must be [rows, Hkv, top_k], got {tuple(topk_idx.shape)}")
    _topk_shapes(topk_idx, None, rows_cap, ckv.num_kv_heads, topk_idx.shape[-1])
    out = _out(out, q, rows_cap, out_dtype)
    workspace, ws_bytes = _workspace(workspace, rows_cap, q, num_splits, "sparse")
    _dev_err(dev_err)
    _same_device(q.device, qo_indptr=qo_indptr, kv_len=kv_len, k=kv.k, block_table=block_table,
                 topk_idx=topk_idx, out=out, workspace=workspace, dev_err=dev_err)
    _call("verify_attention_sparse", family,
          _ptr(q), dtype_code(q.dtype), _ptr(qo_indptr), _ptr(kv_len), B, max_qo_len, q.shape[1],
          C.byref(ckv), _ptr(block_table), block_table.shape[1], block_table.stride(0),
          _ptr(topk_idx), topk_idx.shape[-1], softmax_scale, num_splits, _ptr(workspace),
          ws_bytes, _ptr(out), dtype_code(out.dtype), _ptr(dev_err), _stream(q.device))
    return out


def verify_attention_sparse_select(q: torch.Tensor, qo_indptr: torch.Tensor, kv_len: torch.Tensor,
                                   kv: PagedKV, block_table: torch.Tensor, scores: torch.Tensor, *,
                                   max_qo_len: int, top_k: int, softmax_scale: float,
                                   num_splits: int = 1, workspace: Optional[torch.Tensor] = None,
                                   out: Optional[torch.Tensor] = None, out_dtype=None,
                                   topk_idx: Optional[torch.Tensor] = None,
                                   topk_cnt: Optional[torch.Tensor] = None,
                                   dev_err: Optional[torch.Tensor] = None,
                                   family: int = 0) -> torch.Tensor:
    """Ladder top-k of `scores` and sparse verify attention in one launch; the selection
    is written to `topk_idx` / `topk_cnt` when given."""
    B = _lengths(qo_indptr, kv_len)
    ckv = kv.c()
    rows_cap = B * max_qo_len
    _query(q, rows_cap, ckv.num_kv_heads, ckv.head_dim)
    _block_table(block_table, B)
    _scores_shape(scores, rows_cap, ckv.num_kv_heads, block_table.shape[1])
    _topk_shapes(topk_idx, topk_cnt, rows_cap, ckv.num_kv_heads, top_k)
    out = _out(out, q, rows_cap, out_dtype)
    workspace, ws_bytes = _workspace(workspace, rows_cap, q, num_splits, "sparse")
    _dev_err(dev_err)
    _same_device(q.device, qo_indptr=qo_indptr, kv_len=kv_len, k=kv.k, block_table=block_table,
                 scores=scores, topk_idx=topk_idx, topk_cnt=topk_cnt, out=out,
                 workspace=workspace, dev_err=dev_err)
    _call("verify_attention_sparse_select", family,
          _ptr(q), dtype_code(q.dtype), _ptr(qo_indptr), _ptr(kv_len), B, max_qo_len, q.shape[1],
          C.byref(ckv), _ptr(block_table), block_table.shape[1], block_table.stride(0),
          _ptr(scores), top_k, _ptr(topk_idx), _ptr(topk_cnt), softmax_scale, num_splits,
          _ptr(workspace), ws_bytes, _ptr(out), dtype_code(out.dtype), _ptr(dev_err),
          _stream(q.device))
    return out


def verify_attention_paged(q: torch.Tensor, qo_indptr: torch.Tensor, kv_len: torch.Tensor,
                           kv: PagedKV, block_table: torch.Tensor, *, max_qo_len: int,
                           softmax_scale: float, num_splits: int = 1,
                           workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None, out_dtype=None,
                           dev_err: Optional[torch.Tensor] = None,
                           family: int = 0) -> torch.Tensor:
    """Dense verify attention over every page below each token's ladder bound."""
    B = _lengths(qo_indptr, kv_len)
    ckv = kv.c()
    rows_cap = B * max_qo_len
    _query(q, rows_cap, ckv.num_kv_heads, ckv.head_dim)
    _block_table(block_table, B)
    out = _out(out, q, rows_cap, out_dtype)
    workspace, ws_bytes = _workspace(workspace, rows_cap, q, num_splits, "paged")
    _dev_err(dev_err)
    _same_device(q.device, qo_indptr=qo_indptr, kv_len=kv_len, k=kv.k, block_table=block_table,
                 out=out, workspace=workspace, dev_err=dev_err)
    _call("verify_attention_paged", family,
          _ptr(q), dtype_code(q.dtype), _ptr(qo_indptr), _ptr(kv_len), B, max_qo_len, q.shape[1],
          C.byref(ckv), _ptr(block_table), block_table.shape[1], block_table.stride(0),
          softmax_scale, num_splits, _ptr(workspace), ws_bytes, _ptr(out), dtype_code(out.dtype),
          _ptr(dev_err), _stream(q.device))
    return out


def _new_rows(k_new, v_new, rows_cap, Hkv, d):
    _need(k_new, "k_new")
    _need(v_new, "v_new")
    if v_new.dtype != k_new.dtype:
        raise ValueError("k_new and v_new must share a dtype")
    _rows_at_least(k_new, "k_new", rows_cap, (Hkv, d))
    _rows_at_least(v_new, "v_new", rows_cap, (Hkv, d))


def stage_verify_kv_paged(k_new: torch.Tensor, v_new: torch.Tensor, qo_indptr: torch.Tensor,
                          kv_len: torch.Tensor, kv: PagedKV, block_table: torch.Tensor, *,
                          max_qo_len: int, dev_err: Optional[torch.Tensor] = None) -> None:
    """Write the new tokens' K/V rows [>= B * max_qo_len, Hkv, d] (cache dtype) into
    kv.k / kv.v."""
    B = _lengths(qo_indptr, kv_len)
    ckv = kv.c()
    _new_rows(k_new, v_new, B * max_qo_len, ckv.num_kv_heads, ckv.head_dim)
    _block_table(block_table, B)
    _dev_err(dev_err)
    _same_device(k_new.device, v_new=v_new, qo_indptr=qo_indptr, kv_len=kv_len, k=kv.k,
                 block_table=block_table, dev_err=dev_err)
    L.check(L.load().stage_verify_kv_paged(
        _ptr(k_new), _ptr(v_new), dtype_code(k_new.dtype), _ptr(qo_indptr), _ptr(kv_len), B,
        max_qo_len,
        C.byref(ckv), _ptr(block_table), block_table.shape[1], block_table.stride(0),
        _ptr(dev_err), _stream(k_new.device)))


def stage_verify_kv_view(k_new: torch.Tensor, v_new: torch.Tensor, qo_indptr: torch.Tensor,
                         kv_len: torch.Tensor, view: SubpageView, sub_offsets: torch.Tensor, *,
                         max_qo_len: int, dev_err: Optional[torch.Tensor] = None) -> None:
    """Write the new tokens' K/V rows [>= B * max_qo_len, Hkv, d] into the draft layer
    through the view."""
    B = _lengths(qo_indptr, kv_len)
    _new_rows(k_new, v_new, B * max_qo_len, view.num_kv_heads, view.head_dim)
    _need(sub_offsets, "sub_offsets", torch.int32)
    if sub_offsets.dim() != 3 or sub_offsets.shape[0] != B or sub_offsets.shape[1] != 2:
        raise ValueError(f"sub_offsets must be [B = {B}, 2, max_sub_pages], got "
                         f"{tuple(sub_offsets.shape)}")
    _dev_err(dev_err)
    _same_device(k_new.device, v_new=v_new, qo_indptr=qo_indptr, kv_len=kv_len,
                 sub_offsets=sub_offsets, pool=view.pool, dev_err=dev_err)
    L.check(L.load().stage_verify_kv_view(
        _ptr(k_new), _ptr(v_new), dtype_code(k_new.dtype), _ptr(qo_indptr), _ptr(kv_len), B,
        max_qo_len, C.byref(view.c), _ptr(sub_offsets), sub_offsets.shape[-1], _ptr(dev_err),
        _stream(k_new.device)))


def hnd_head_slice_descriptors(*, token_groups: int, src_heads: int, src_head_begin: int,
                               dst_heads: int, dst_head_begin: int, num_heads: int,
                               head_dim: int, kv_dtype, src_page_offsets, dst_page_offsets,
                               page_tokens: int = 128) -> np.ndarray:
    """Host-side mapper: int64 [num_pages * token_groups, 3] (src offset, dst offset,
    bytes), one row per (page, token group)."""
    src = np.ascontiguousarray(src_page_offsets, dtype=np.int64)
    dst = np.ascontiguousarray(dst_page_offsets, dtype=np.int64)
    n = src.size
    if dst.size != n:
        raise ValueError(f"{n} source pages but {dst.size} destination pages")
    out = np.zeros((max(n * token_groups, 1), 3), dtype=np.int64)
    count = C.c_int32(0)
    L.check(L.load().hnd_head_slice_descriptors(
        token_groups, src_heads, src_head_begin, dst_heads, dst_head_begin, num_heads, head_dim,
        dtype_code(kv_dtype), page_tokens, src.ctypes.data, dst.ctypes.data, n,
        out.ctypes.data, out.shape[0], C.byref(count)))
    return out[:count.value]


def copy_descriptors(src: torch.Tensor, dst: torch.Tensor, descs: torch.Tensor, *,
                     dev_err: Optional[torch.Tensor] = None) -> None:
    """Execute byte-range copies (descs: int64 [n, 3] on the device) from src into dst."""
    _need(descs, "descs", torch.int64)
    if descs.dim() != 2 or descs.shape[1] != 3:
        raise ValueError(f"descs must be [n, 3], got {tuple(descs.shape)}")
    _need(src, "src")
    _need(dst, "dst")
    _dev_err(dev_err)
    _same_device(dst.device, src=src, descs=descs, dev_err=dev_err)
    L.check(L.load().copy_descriptors(
        _ptr(src), src.numel() * src.element_size(), _ptr(dst), dst.numel() * dst.element_size(),
        _ptr(descs), descs.shape[0], _ptr(dev_err), _stream(dst.device)))


def greedy_accept_workspace_bytes(B: int, max_qo_len: int, vocab: int, dtype) -> int:
    return int(L.load().sdv_greedy_accept_workspace_bytes(B, max_qo_len, vocab, dtype_code(dtype)))


def greedy_accept(logits: torch.Tensor, tokens: torch.Tensor, qo_indptr: torch.Tensor,
                  kv_len: torch.Tensor, *, max_qo_len: int,
                  dev_err: Optional[torch.Tensor] = None, outs=None,
                  workspace: Optional[torch.Tensor] = None):
    """Returns (targets [B*max_qo_len], accept [B], emitted [B, max_qo_len], new_kv_len [B]);
    `outs` may pass those four int32 tensors preallocated, `workspace` a byte tensor of
    greedy_accept_workspace_bytes(...) or more.  Target rows past qo_indptr[B] are left
    as they were.  logits [rows, vocab] and tokens [rows] hold the verify rows
    (rows = qo_indptr[B])."""
    B = _lengths(qo_indptr, kv_len)
    _need(logits, "logits")
    _need(tokens, "tokens", torch.int32)
    if logits.dim() != 2:
        raise ValueError(f"logits must be [rows, vocab], got {tuple(logits.shape)}")
    if tokens.numel() != logits.shape[0]:
        raise ValueError(f"tokens holds {tokens.numel()} rows, logits {logits.shape[0]}")
    dev = logits.device
    vocab = logits.shape[-1]
    rows_cap = B * max_qo_len
    if outs is None:
        outs = (torch.empty(rows_cap, dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty((B, max_qo_len), dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev))
    targets, accept, emitted, new_kv = outs
    for name, t, n in (("targets", targets, rows_cap), ("accept", accept, B),
                       ("emitted", emitted, rows_cap), ("new_kv_len", new_kv, B)):
        _need(t, name, torch.int32)
        if t.numel() < n:
            raise ValueError(f"{name} must hold {n} int32, got {t.numel()}")
    if workspace is None:
        need = greedy_accept_workspace_bytes(B, max_qo_len, vocab, logits.dtype)
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace")
    _dev_err(dev_err)
    _same_device(dev, tokens=tokens, qo_indptr=qo_indptr, kv_len=kv_len, workspace=workspace,
                 targets=targets, accept=accept, emitted=emitted, new_kv_len=new_kv,
                 dev_err=dev_err)
    L.check(L.load().greedy_accept(
        _ptr(logits), dtype_code(logits.dtype), vocab, _ptr(tokens), _ptr(qo_indptr),
        _ptr(kv_len), B, max_qo_len, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(targets), _ptr(accept), _ptr(emitted), _ptr(new_kv), _ptr(dev_err), _stream(dev)))
    return targets, accept, emitted, new_kv


def lse_combine(partial_out: torch.Tensor, partial_lse: torch.Tensor, *, out_dtype=torch.float32,
                out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                want_lse: bool = False):
    """partial_out [S, rows, H, d] float32, partial_lse [S, rows, H] float32."""
    _need(partial_out, "partial_out", torch.float32)
    _need(partial_lse, "partial_lse", torch.float32)
    if partial_out.dim() != 4:
        raise ValueError(f"partial_out must be [S, rows, H, d], got {tuple(partial_out.shape)}")
    S, rows, H, d = partial_out.shape
    if tuple(partial_lse.shape) != (S, rows, H):
        raise ValueError(f"partial_lse must be [{S}, {rows}, {H}], got {tuple(partial_lse.shape)}")
    if out is None:
        out = torch.empty((rows, H, d), dtype=out_dtype, device=partial_out.device)
    _need(out, "out")
    if out.dtype not in _OUT_DT:
        raise TypeError(f"out must be float32 or bfloat16, got {out.dtype}")
    _rows_at_least(out, "out", rows, (H, d))
    if lse_out is None and want_lse:
        lse_out = torch.empty((rows, H), dtype=torch.float32, device=partial_out.device)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32)
        _rows_at_least(lse_out, "lse_out", rows, (H,))
    _same_device(partial_out.device, partial_lse=partial_lse, out=out, lse_out=lse_out)
    L.check(L.load().lse_combine(_ptr(partial_out), _ptr(partial_lse), S, rows, H, d, _ptr(out),
                                 dtype_code(out.dtype), _ptr(lse_out),
                                 _stream(partial_out.device)))
    return (out, lse_out) if want_lse else out


def fill_u32(dst: torch.Tensor, pattern: int = 0) -> None:
    _need(dst, "dst")
    L.check(L.load().sdv_fill_u32(_ptr(dst), dst.numel() * dst.element_size(), pattern,
                                  _stream(dst.device)))


def read_units_probe(base: torch.Tensor, units: torch.Tensor, unit_bytes: int, sink: torch.Tensor,
                     blocks: int) -> None:
    """Streaming read of the listed unit_bytes units of base (measurement helper); units:
    int64 device tensor of unit indices; sink: int32 [>= blocks]."""
    _need(units, "units", torch.int64)
    _need(sink, "sink", torch.int32)
    if sink.numel() < blocks:
        raise ValueError(f"sink must hold {blocks} words")
    _same_device(base.device, units=units, sink=sink)
    L.check(L.load().sdv_read_units_probe(_ptr(base), base.numel() * base.element_size(), _ptr(units),
                                          units.numel(), unit_bytes, _ptr(sink), blocks,
                                          _stream(base.device)))


def read_probe(src: torch.Tensor, sink: torch.Tensor, blocks: int) -> None:
    """Streaming read of all of src (measurement helper); sink: int32 [>= blocks]."""
    _need(sink, "sink", torch.int32)
    if sink.numel() < blocks:
        raise ValueError(f"sink must hold {blocks} words")
    _same_device(src.device, sink=sink)
    L.check(L.load().sdv_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                    blocks, _stream(src.device)))
