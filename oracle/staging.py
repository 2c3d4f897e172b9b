"""Ladder KV slot staging: the verify step writes the K/V of its qo_len new tokens
into the paged cache before attention reads them.

[PR3] MSA verify commit: KV slot staging generalises to the causal ladder — the
qo_len = 1 + draft_len tokens of a request are appended together, token t at logical
position kv_len - qo_len + t (kv_len counts them), across page boundaries.  The same
commit's overlap correction: a correction that shortens a row across a page boundary
must re-stage with the corrected lengths, and no other row's pages may move — here each
request has its own block-table row, so staging depends only on that request's
lengths.

Addressing (the pages' layouts, as in view.py): an ordinary head-major page holds
position j of its request at [page = block_table[r][j // 128], head, j % 128, :]; the
draft layer's P32 view holds it at P32 page offsets[r][0][j // 32] (K; V four P32 pages
on), token j % 32, element ((x * Hkv + h) * 32 + j % 32) * d + c from the view root.

Values are copied as stored (no conversion): new rows arrive in the pool's storage
format.  The functions return updated copies and leave their inputs alone.
"""
import numpy as np

from .view import subpage_offsets

PAGE = 128
SUB = 32


def stage_paged(k_pool, v_pool, k_new, v_new, qo_indptr, kv_len, block_table, page=PAGE):
    """k_pool, v_pool [num_pages, Hkv, 128, d]; k_new, v_new [rows, Hkv, d] (rows in
    qo_indptr order).  Returns (k_pool', v_pool')."""
    kp, vp = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    for r in range(len(kv_len)):
        a, b = int(qo_indptr[r]), int(qo_indptr[r + 1])
        qo, kv = b - a, int(kv_len[r])
        for t in range(qo):
            j = kv - qo + t
            pg = int(block_table[r][j // page])
            kp[pg, :, j % page, :] = k_new[a + t]
            vp[pg, :, j % page, :] = v_new[a + t]
    return kp, vp


def stage_view(pool_flat, root_elem, k_new, v_new, qo_indptr, kv_len, block_table, slot_stride,
               num_kv_heads, head_dim):
    """pool_flat: 1-D stored elements of the whole flat P128 pool; the view is rooted at
    element root_elem; block_table [B, W] of P128 slot ids.  Returns pool_flat'."""
    out = np.array(pool_flat, copy=True)
    offs = subpage_offsets(block_table, slot_stride)
    H, d = num_kv_heads, head_dim
    for r in range(len(kv_len)):
        a, b = int(qo_indptr[r]), int(qo_indptr[r + 1])
        qo, kv = b - a, int(kv_len[r])
        for t in range(qo):
            j = kv - qo + t
            for kind, src in ((0, k_new), (1, v_new)):
                x = int(offs[r, kind, j // SUB])
                for h in range(H):
                    e0 = root_elem + ((x * H + h) * SUB + j % SUB) * d
                    out[e0:e0 + d] = src[a + t, h]
    return out
