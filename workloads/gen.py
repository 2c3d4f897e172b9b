"""Seeded synthetic inputs for the verify step, shared by the CPU oracle's tests and
the GPU path.

This module draws random numbers and lays out buffers; it computes nothing of the
method (no ladder, no view index arithmetic, no scores, no attention).  Both sides
receive the same bytes from here.

Layouts produced:
  * q:           [sum(qo), Hq, d], row = qo_indptr[r] + t, query head hq.
  * dense pool:  flat array of 128-token pages, page shape [4, Hkv, 32, d] (four
                 head-major 32-token groups).  Slot s owns pages
                 [s * stride, (s + 1) * stride); the draft layer's K page is in-slot
                 page `root_page` and its V page the next one.  Slot 0 is reserved
                 and never assigned; block-table padding is 0.
  * sparse pool: K and V arrays [num_pages, Hkv, 128, d] (ordinary head-major page).
  * block table: int32 [B, capacity_pages]; request r's pages are a run of a seeded
                 random permutation of the physical pages (or slots), padding 0.

The fp8 storage uses the library conversion torch.float8_e4m3fn with one fp32
per-tensor scale = amax / 448 (the format's largest finite value).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import PAGE, SUB_PAGE, VerifyWorkload

FP8_MAX = 448.0
_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


def seed_for(workload: VerifyWorkload, base: int = 1000) -> int:
    names = ("tiny_fp32", "dense_bf16", "sparse_bf16", "long_fp8", "ragged_mixed", "paged_bf16")
    idx = names.index(workload.name) + 1 if workload.name in names else 99
    return base + idx


def draw_lengths(w: VerifyWorkload, seed: int):
    """Per-request (qo_len, kv_len), int64 numpy arrays, from a seeded PCG64 stream."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B = w.batch
    if isinstance(w.qo, int):
        qo = np.full(B, w.qo, dtype=np.int64)
    else:
        _, lo, hi = w.qo
        qo = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    kind = w.kv[0]
    if kind == "list":
        vals = np.asarray(w.kv[1], dtype=np.int64)
        assert len(vals) == B
        kv = vals.copy()
    elif kind == "uniform":
        kv = rng.integers(w.kv[1], w.kv[2] + 1, size=B).astype(np.int64)
    elif kind == "fixed":
        kv = np.full(B, w.kv[1], dtype=np.int64)
    elif kind == "lognormal":
        _, median, sigma, lo, hi, cross_frac = w.kv
        raw = np.exp(np.log(median) + sigma * rng.standard_normal(B))
        kv = np.clip(np.rint(raw), lo, hi).astype(np.int64)
        kv = np.maximum(kv, qo)
        # Rows deliberately crossing a page boundary: a quarter of the rows with
        # qo >= 2 get kv mod 128 in [1, qo - 1].
        cand = np.nonzero(qo >= 2)[0]
        pick = rng.random(len(cand)) < cross_frac
        for r in cand[pick]:
            base = PAGE * max(1, int(kv[r]) // PAGE)
            if base + int(qo[r]) - 1 > hi:
                base -= PAGE
            kv[r] = base + int(rng.integers(1, int(qo[r])))
    else:
        raise ValueError(kind)
    if w.kv_capacity is not None:
        kv = np.minimum(kv, w.kv_capacity)
    assert np.all(kv >= qo) and np.all(qo >= 1)
    return qo, kv


def _values(w: VerifyWorkload, shape, gen: torch.Generator, device) -> torch.Tensor:
    if w.values == "int4":
        return torch.randint(-4, 5, shape, generator=gen, device=device).to(torch.float32)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _store(x: torch.Tensor, dtype: str):
    """Cast float32 values to the storage dtype; returns (tensor, scale)."""
    if dtype == "fp8":
        amax = float(x.abs().max())
        scale = amax / FP8_MAX if amax > 0 else 1.0
        return (x / scale).to(torch.float8_e4m3fn), scale
    return x.to(_TORCH_DTYPE[dtype]), 1.0


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


@dataclass
class Lengths:
    qo: np.ndarray
    kv: np.ndarray

    @property
    def qo_indptr(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.qo)]).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(self.qo.sum())


@dataclass
class DenseCase:
    w: VerifyWorkload
    lengths: Lengths
    q: torch.Tensor              # [sum(qo), Hq, d]
    qo_indptr: torch.Tensor      # int32 [B + 1]
    kv_len: torch.Tensor         # int32 [B]
    pool: torch.Tensor           # [num_slots * stride, 4, Hkv, 32, d]
    block_table: torch.Tensor    # int32 [B, max_blocks], P128 slot ids
    num_slots: int
    k_scale: float
    v_scale: float
    softmax_scale: float


@dataclass
class SparseCase:
    w: VerifyWorkload
    lengths: Lengths
    q: torch.Tensor              # [sum(qo), Hq, d]
    qo_indptr: torch.Tensor
    kv_len: torch.Tensor
    k_pool: torch.Tensor         # [num_pages, Hkv, 128, d]
    v_pool: torch.Tensor
    block_table: torch.Tensor    # int32 [B, max_pages]
    num_pages: int
    k_scale: float
    v_scale: float
    softmax_scale: float


def _common(w: VerifyWorkload, seed: int, device):
    qo, kv = draw_lengths(w, seed)
    lengths = Lengths(qo=qo, kv=kv)
    gq = _gen(seed * 7 + 1, device)
    q32 = _values(w, (lengths.total_q, w.num_q_heads, w.head_dim), gq, device)
    q = q32.to(_TORCH_DTYPE[w.q_dtype])
    qo_indptr = torch.from_numpy(lengths.qo_indptr).to(device)
    kv_len = torch.from_numpy(kv.astype(np.int32)).to(device)
    return lengths, q, qo_indptr, kv_len


def _block_table(n_pages_per_req, capacity_pages, ids: np.ndarray) -> np.ndarray:
    B = len(n_pages_per_req)
    bt = np.zeros((B, capacity_pages), dtype=np.int32)
    off = 0
    for r, n in enumerate(n_pages_per_req):
        bt[r, :n] = ids[off:off + n]
        off += n
    return bt


def make_dense_case(w: VerifyWorkload, seed: Optional[int] = None, device="cpu",
                    poison: bool = False) -> DenseCase:
    """Draft-layer case: a flat pool of P128 pages read through the P32 view."""
    seed = seed_for(w) if seed is None else seed
    lengths, q, qo_indptr, kv_len = _common(w, seed, device)
    n_pages = [-(-int(k) // PAGE) for k in lengths.kv]
    num_slots = 1 + sum(n_pages) + w.spare_pages          # slot 0 reserved
    rng = np.random.Generator(np.random.PCG64(seed * 7 + 2))
    slots = rng.permutation(np.arange(1, num_slots, dtype=np.int32))
    bt = _block_table(n_pages, w.max_pages(), slots)
    stride = w.slot_stride
    assert 0 <= w.root_page and w.root_page + 1 < stride
    shape = (num_slots * stride, 4, w.num_kv_heads, SUB_PAGE, w.head_dim)
    gp = _gen(seed * 7 + 3, device)
    vals = _values(w, shape, gp, device)
    if poison:
        # Pages other than the draft layer's K/V pages of assigned slots hold NaN.
        keep = torch.zeros(num_slots * stride, dtype=torch.bool, device=device)
        used = torch.from_numpy(np.sort(slots[:sum(n_pages)]).astype(np.int64)).to(device)
        keep[used * stride + w.root_page] = True
        keep[used * stride + w.root_page + 1] = True
        vals[~keep] = float("nan")
    # K and V pages share one pool tensor, hence one scale (the pool is one tensor).
    pool, scale = _store(vals, w.kv_dtype) if not poison else _store_poisoned(vals, w.kv_dtype)
    return DenseCase(w=w, lengths=lengths, q=q, qo_indptr=qo_indptr, kv_len=kv_len,
                     pool=pool, block_table=torch.from_numpy(bt).to(device),
                     num_slots=num_slots, k_scale=scale, v_scale=scale,
                     softmax_scale=1.0 / float(np.sqrt(w.head_dim)))


def _store_poisoned(vals: torch.Tensor, dtype: str):
    if dtype == "fp8":
        finite = torch.isfinite(vals)
        amax = float(vals[finite].abs().max())
        scale = amax / FP8_MAX
        out = torch.where(finite, vals / scale, vals).to(torch.float8_e4m3fn)
        return out, scale
    return vals.to(_TORCH_DTYPE[dtype]), 1.0


def make_sparse_case(w: VerifyWorkload, seed: Optional[int] = None, device="cpu",
                     poison: bool = False) -> SparseCase:
    """Target-layer case: K and V arrays of ordinary head-major P128 pages."""
    seed = seed_for(w) if seed is None else seed
    lengths, q, qo_indptr, kv_len = _common(w, seed, device)
    n_pages = [-(-int(k) // PAGE) for k in lengths.kv]
    num_pages = sum(n_pages) + w.spare_pages
    rng = np.random.Generator(np.random.PCG64(seed * 7 + 4))
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = _block_table(n_pages, w.max_pages(), perm)
    shape = (num_pages, w.num_kv_heads, PAGE, w.head_dim)
    gk = _gen(seed * 7 + 5, device)
    kvals = _values(w, shape, gk, device)
    gv = _gen(seed * 7 + 6, device)
    vvals = _values(w, shape, gv, device)
    if poison:
        keep = torch.zeros(num_pages, dtype=torch.bool, device=device)
        keep[torch.from_numpy(perm[:sum(n_pages)].astype(np.int64)).to(device)] = True
        kvals[~keep] = float("nan")
        vvals[~keep] = float("nan")
        k_pool, k_scale = _store_poisoned(kvals, w.kv_dtype)
        v_pool, v_scale = _store_poisoned(vvals, w.kv_dtype)
    else:
        k_pool, k_scale = _store(kvals, w.kv_dtype)
        v_pool, v_scale = _store(vvals, w.kv_dtype)
    del kvals, vvals
    return SparseCase(w=w, lengths=lengths, q=q, qo_indptr=qo_indptr, kv_len=kv_len,
                      k_pool=k_pool, v_pool=v_pool, block_table=torch.from_numpy(bt).to(device),
                      num_pages=num_pages, k_scale=k_scale, v_scale=v_scale,
                      softmax_scale=1.0 / float(np.sqrt(w.head_dim)))


def raw_numpy(t: torch.Tensor) -> np.ndarray:
    """The stored bytes as a numpy array: float32 as float32, bf16 as uint16 bit
    patterns, fp8 as uint8 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    raise TypeError(t.dtype)


DTYPE_NAME = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}


@dataclass
class AcceptCase:
    lengths: Lengths
    logits: torch.Tensor          # [sum(qo), vocab], f32 or bf16
    tokens: torch.Tensor          # int32 [sum(qo)]: row 0 the last accepted token, then drafts
    qo_indptr: torch.Tensor
    kv_len: torch.Tensor
    planted: np.ndarray           # int64 [sum(qo)]: the index given the margin in each row


def make_accept_case(w: VerifyWorkload, vocab: int, p_match: float = 0.8,
                     dtype: torch.dtype = torch.bfloat16, tie_rows: float = 0.1,
                     nan_rows: float = 0.0, seed: Optional[int] = None,
                     device=None) -> AcceptCase:
    """Target logits for the verify rows of workload w's lengths, with known structure:
    each row holds N(0, 1) values plus one planted index raised 2.0 above the row's
    largest draw; a fraction of rows copies that value to a second, random index (two
    equal maxima); a fraction gets NaN at random places.  Row t >= 1 of a request holds
    the planted index of row t - 1 with probability p_match, else another random token
    (only the drawing is done here: which token the target picks is left to the code
    under test)."""
    seed = seed_for(w, 3000) if seed is None else seed
    qo_, kv_ = draw_lengths(w, seed)
    lengths = Lengths(qo=qo_, kv=kv_)
    rows = lengths.total_q
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, vocab)).astype(np.float32)
    planted = rng.integers(0, vocab, size=rows)
    top = x.max(axis=1) + 2.0
    x[np.arange(rows), planted] = top
    tie = rng.random(rows) < tie_rows
    second = rng.integers(0, vocab, size=rows)
    x[tie, second[tie]] = top[tie]
    if nan_rows > 0:
        nanr = rng.random(rows) < nan_rows
        cols = rng.integers(0, vocab, size=(rows, 4))
        for r_ in np.nonzero(nanr)[0]:
            x[r_, cols[r_]] = np.nan
    tokens = rng.integers(0, vocab, size=rows)
    ind = lengths.qo_indptr
    for r in range(w.batch):
        for t in range(1, int(lengths.qo[r])):
            row = ind[r] + t
            if rng.random() < p_match:
                tokens[row] = planted[row - 1]
    logits = torch.from_numpy(x).to(dtype)
    dev = device if device is not None else torch.device("cpu")
    return AcceptCase(lengths=lengths, logits=logits.to(dev),
                      tokens=torch.from_numpy(tokens.astype(np.int32)).to(dev),
                      qo_indptr=torch.from_numpy(ind.astype(np.int32)).to(dev),
                      kv_len=torch.from_numpy(lengths.kv.astype(np.int32)).to(dev),
                      planted=planted)
