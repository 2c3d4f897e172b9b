"""Helpers shared by the GPU parity tests: run a generated case through the library
and through the oracle, and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import speculative_decode_verify_p128_amd as sdv
import workloads as W
from workloads import raw_numpy

DEV = torch.device("cuda:0")


def q_capacity(q: torch.Tensor, rows: int) -> torch.Tensor:
    """q on the GPU with at least `rows` rows (the B * max_qo_len capacity the library
    addresses); rows past the batch's tokens are zero and never read."""
    out = torch.zeros((max(rows, q.shape[0]),) + tuple(q.shape[1:]), dtype=q.dtype, device=DEV)
    out[:q.shape[0]] = q.to(DEV)
    return out


def tol_ok(got: np.ndarray, ref: np.ndarray, dtype: str):
    """fp32: |gpu - ref| <= 1e-4 |ref| + 1e-5 elementwise; bf16/fp8: max-abs <= 2e-2."""
    got = np.asarray(got, dtype=np.float64)
    if dtype == "f32":
        bad = np.abs(got - ref) > 1e-4 * np.abs(ref) + 1e-5
    else:
        bad = np.abs(got - ref) > 2e-2
    bad |= ~np.isfinite(got)
    return not bad.any(), float(np.nanmax(np.abs(got - ref))) if got.size else 0.0


class SparseRun:
    def __init__(self, c: W.SparseCase):
        self.c = c
        w = c.w
        self.kv = sdv.PagedKV(c.k_pool.to(DEV), c.v_pool.to(DEV), c.k_scale, c.v_scale)
        self.q = q_capacity(c.q, w.batch * w.max_qo())
        self.qo_indptr = c.qo_indptr.to(DEV)
        self.kv_len = c.kv_len.to(DEV)
        self.bt = c.block_table.to(DEV)
        self.max_qo = w.max_qo()
        self.n = c.lengths.total_q

    def scores(self, dev_err=None):
        return sdv.proxy_page_scores(self.q, self.qo_indptr, self.kv_len, self.kv, self.bt,
                                     max_qo_len=self.max_qo, dev_err=dev_err)

    def topk(self, scores, top_k=None, dev_err=None):
        return sdv.ladder_topk_pages(scores, self.qo_indptr, self.kv_len, max_qo_len=self.max_qo,
                                     top_k=top_k or self.c.w.top_k, want_count=True,
                                     dev_err=dev_err)

    def attend(self, idx, num_splits=1, dev_err=None, family=0):
        return sdv.verify_attention_sparse(self.q, self.qo_indptr, self.kv_len, self.kv, self.bt,
                                           idx, max_qo_len=self.max_qo,
                                           softmax_scale=self.c.softmax_scale,
                                           num_splits=num_splits, dev_err=dev_err, family=family)


class PagedRun(SparseRun):
    def attend_paged(self, num_splits=1, dev_err=None, family=0):
        return sdv.verify_attention_paged(self.q, self.qo_indptr, self.kv_len, self.kv, self.bt,
                                          max_qo_len=self.max_qo,
                                          softmax_scale=self.c.softmax_scale,
                                          num_splits=num_splits, dev_err=dev_err, family=family)


def paged_oracle(c: W.SparseCase, requests=None):
    w = c.w
    return oracle.paged_verify_case(
        raw_numpy(c.q), w.q_dtype, c.qo_indptr.numpy(), c.lengths.kv, raw_numpy(c.k_pool),
        raw_numpy(c.v_pool), w.kv_dtype, c.block_table.numpy(), c.k_scale, c.v_scale,
        c.softmax_scale, requests=requests)


def sparse_oracle(c: W.SparseCase, requests=None, top_k=None):
    w = c.w
    return oracle.sparse_verify_case(
        raw_numpy(c.q), w.q_dtype, c.qo_indptr.numpy(), c.lengths.kv, raw_numpy(c.k_pool),
        raw_numpy(c.v_pool), w.kv_dtype, c.block_table.numpy(), c.k_scale, c.v_scale,
        top_k or w.top_k, c.softmax_scale, w.max_pages(), requests=requests)


class DenseRun:
    def __init__(self, c: W.DenseCase):
        self.c = c
        w = c.w
        self.pool = c.pool.to(DEV)
        self.q = q_capacity(c.q, w.batch * w.max_qo())
        self.qo_indptr = c.qo_indptr.to(DEV)
        self.kv_len = c.kv_len.to(DEV)
        self.bt = c.block_table.to(DEV)
        self.max_qo = w.max_qo()
        self.n = c.lengths.total_q

    def view(self, dev_err=None):
        w = self.c.w
        return sdv.kv_subpage_view_init(self.pool[w.root_page], self.bt,
                                        num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                        slot_stride=w.slot_stride, num_slots=self.c.num_slots,
                                        k_scale=self.c.k_scale, v_scale=self.c.v_scale,
                                        pool_index_scale=w.pool_index_scale, dev_err=dev_err)

    def attend(self, view, offs, num_splits=1, dev_err=None, family=0):
        return sdv.verify_attention_dense(self.q, self.qo_indptr, self.kv_len, view, offs,
                                          max_qo_len=self.max_qo,
                                          softmax_scale=self.c.softmax_scale,
                                          num_splits=num_splits, dev_err=dev_err, family=family)


def dense_oracle(c: W.DenseCase, requests=None):
    w = c.w
    page_elems = 4 * w.num_kv_heads * 32 * w.head_dim
    return oracle.dense_verify_case(
        raw_numpy(c.q), w.q_dtype, c.qo_indptr.numpy(), c.lengths.kv,
        raw_numpy(c.pool).reshape(-1), w.kv_dtype, w.root_page * page_elems,
        c.block_table.numpy(), w.slot_stride, w.num_kv_heads, w.head_dim, c.k_scale,
        c.v_scale, c.softmax_scale, requests=requests)


def rows_of(c, requests):
    ind = c.qo_indptr.numpy()
    return np.concatenate([np.arange(ind[r], ind[r + 1]) for r in requests])


def out_numpy(t: torch.Tensor) -> np.ndarray:
    return t.double().cpu().numpy()
