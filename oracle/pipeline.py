"""Whole-path oracle for a batch: dense draft-layer verify through the P32 view, and
the sparse target-layer path (proxy scores -> ladder top-k -> sparse attention).

Inputs are plain NumPy arrays of the stored bytes (float32 values, bf16 bit patterns
as uint16, fp8 bit patterns as uint8) plus the per-tensor scales, so the same bytes
the GPU receives are decoded here from the formats' definitions.  Requests are
processed one at a time (bounded memory); `requests` restricts the work to a sample.

Sources: [PR3] MSA verify commit (ladder, proxy pass, per-token top-k, sparse pass);
[PR17835] Description and "Grouped-HND draft KV transfer" (P32 view of P128 pages);
[PR18066] view-scale commit (root, stride, V = K + 1 page).
"""
import numpy as np

from .attention import dense_verify_request, sparse_verify_request
from .fp8 import decode_store
from .proxy import proxy_scores_request
from .topk import ladder_topk_request
from .view import gather_hnd, gather_subpage_view, subpage_offsets



def _q_values(q_raw, q_dtype):
    return decode_store(q_raw, q_dtype)                 # float32 values


def request_kv_dense(pool_flat_raw, kv_dtype, root_elem, block_table_row, slot_stride,
                     kv_len, num_kv_heads, head_dim):
    """Unscaled float32 K, V [kv_len, Hkv, d] of one request through the P32 view."""
    offs = subpage_offsets(np.asarray(block_table_row)[None, :], slot_stride)[0]
    root_flat = pool_flat_raw[root_elem:]
    k_raw, v_raw = gather_subpage_view(root_flat, offs, int(kv_len), num_kv_heads, head_dim)
    return decode_store(k_raw, kv_dtype), decode_store(v_raw, kv_dtype)


def request_kv_sparse(k_pool_raw, v_pool_raw, kv_dtype, block_table_row, kv_len):
    """Unscaled float32 K, V [kv_len, Hkv, d] of one request from head-major pages."""
    k = gather_hnd(k_pool_raw, block_table_row, int(kv_len))
    v = gather_hnd(v_pool_raw, block_table_row, int(kv_len))
    return decode_store(k, kv_dtype), decode_store(v, kv_dtype)


def dense_verify_case(q_raw, q_dtype, qo_indptr, kv_len, pool_flat_raw, kv_dtype, root_elem,
                      block_table, slot_stride, num_kv_heads, head_dim, k_scale, v_scale,
                      softmax_scale, requests=None):
    """out [sum(qo), Hq, d] float64; rows of requests outside `requests` stay NaN."""
    q = _q_values(q_raw, q_dtype)
    out = np.full(q.shape, np.nan)
    B = len(kv_len)
    for r in (range(B) if requests is None else requests):
        a, b = int(qo_indptr[r]), int(qo_indptr[r + 1])
        k, v = request_kv_dense(pool_flat_raw, kv_dtype, root_elem, block_table[r], slot_stride,
                                kv_len[r], num_kv_heads, head_dim)
        out[a:b] = dense_verify_request(q[a:b].astype(np.float64), k.astype(np.float64) * k_scale,
                                        v.astype(np.float64) * v_scale, int(kv_len[r]),
                                        softmax_scale)
    return out


def paged_verify_case(q_raw, q_dtype, qo_indptr, kv_len, k_pool_raw, v_pool_raw, kv_dtype,
                      block_table, k_scale, v_scale, softmax_scale, requests=None):
    """Dense verify attention over ordinary head-major P128 pages: the target's dense
    layers, whose attention takes a ladder mask ([PR3] MSA verify commit: dense layers
    0-2 get a ladder SDPA mask, the old math at qo_len = 1).  K/V of a request come
    from its block table (position j in page block_table[r][j // 128], token j % 128).
    out [sum(qo), Hq, d] float64; rows of requests outside `requests` stay NaN."""
    q = _q_values(q_raw, q_dtype)
    out = np.full(q.shape, np.nan)
    B = len(kv_len)
    for r in (range(B) if requests is None else requests):
        a, b = int(qo_indptr[r]), int(qo_indptr[r + 1])
        kvr = int(kv_len[r])
        k, v = request_kv_sparse(k_pool_raw, v_pool_raw, kv_dtype, block_table[r], kvr)
        out[a:b] = dense_verify_request(q[a:b].astype(np.float64), k.astype(np.float64) * k_scale,
                                        v.astype(np.float64) * v_scale, kvr, softmax_scale)
    return out


def sparse_verify_case(q_raw, q_dtype, qo_indptr, kv_len, k_pool_raw, v_pool_raw, kv_dtype,
                       block_table, k_scale, v_scale, top_k, softmax_scale, max_pages,
                       requests=None):
    """Returns dict with
         scores [sum(qo), Hkv, max_pages] float32 (NaN beyond each request's pages),
         topk   [sum(qo), Hkv, top_k] int64 (-1 padded), count [sum(qo), Hkv],
         out    [sum(qo), Hq, d] float64;
       rows of requests outside `requests` stay NaN / -2."""
    q = _q_values(q_raw, q_dtype)
    R, Hq, d = q.shape
    Hkv = k_pool_raw.shape[1]
    scores = np.full((R, Hkv, max_pages), np.nan, dtype=np.float32)
    topk = np.full((R, Hkv, top_k), -2, dtype=np.int64)
    count = np.full((R, Hkv), -2, dtype=np.int64)
    out = np.full((R, Hq, d), np.nan)
    B = len(kv_len)
    for r in (range(B) if requests is None else requests):
        a, b = int(qo_indptr[r]), int(qo_indptr[r + 1])
        kvr = int(kv_len[r])
        k, v = request_kv_sparse(k_pool_raw, v_pool_raw, kv_dtype, block_table[r], kvr)
        s = proxy_scores_request(q[a:b], k, kvr)                     # [qo, Hkv, n_pages]
        scores[a:b, :, :s.shape[2]] = s
        idx, cnt = ladder_topk_request(s, kvr, top_k)
        topk[a:b] = idx
        count[a:b] = cnt
        out[a:b] = sparse_verify_request(q[a:b].astype(np.float64), k.astype(np.float64) * k_scale,
                                         v.astype(np.float64) * v_scale, kvr, idx, softmax_scale)
    return {"scores": scores, "topk": topk, "count": count, "out": out}
