"""Paged-KV addressing: the non-owning 32-token sub-page view of the draft layer's
128-token pages, ordinary head-major pages of the target layers, and the head-slice
transfer descriptors of a grouped page.

Facts used, from the pages:
  * [PR17835] Description: target KV uses 128-token pages, the Eagle3 drafter
    consumes 32-token pages, and a non-owning sub-page view bridges the two.
  * [PR17835] Root causes and fixes, item 2 (Grouped-HND draft KV transfer): the P32
    view reads a P128 physical page as four independent head-major token groups,
    logically [group = 4, local_head, 32, head_dim]; an ordinary head-major page is
    [local_head, 128, head_dim].  A mapper that emits one contiguous head slice per
    page is right only in the first 32-token group; the fix emits one descriptor per
    (layer, K/V, token group).
  * [PR18066] view-scale commit: the view is rooted at the draft layer's K page; the
    layer-local stride puts slot s's K at s * stride and its V at s * stride + 1
    (in 128-token pages from the root); that stride is the view's index scale and
    the pool's own page-index scale is not used.
  * [PR18066] dead-code commit: block-table padding is kept as is and addresses
    valid slot-0 memory.

Reading: P32 page index x counts 32-token pages from the view root, so P128 page
(s * stride) holds P32 pages 4 * s * stride + g for groups g = 0..3 and the V page is
4 P32 pages further on.  Element (x, head h, token o, channel c) sits at
((x * Hkv + h) * 32 + o) * d + c elements from the root.
"""
import numpy as np

SUB = 32
GROUPS = 4


def subpage_offsets(block_table: np.ndarray, slot_stride: int) -> np.ndarray:
    """[B, 2, 4 * W] int64 P32-page indices (K row 0, V row 1) from a [B, W] table of
    P128 slot ids.  Sub-page i of request r lies in slot block_table[r, i // 4],
    token group i % 4; padding entries (slot 0) map like any other slot."""
    bt = np.asarray(block_table, dtype=np.int64)
    B, W = bt.shape
    out = np.empty((B, 2, GROUPS * W), dtype=np.int64)
    for r in range(B):
        for i in range(GROUPS * W):
            slot = bt[r, i // GROUPS]
            k_index = slot * slot_stride * GROUPS + i % GROUPS
            out[r, 0, i] = k_index
            out[r, 1, i] = k_index + GROUPS
    return out


def gather_subpage_view(root_flat: np.ndarray, offsets_row: np.ndarray, kv_len: int,
                        num_kv_heads: int, head_dim: int):
    """Logical K and V, each [kv_len, Hkv, d], of one request read through the view.

    root_flat: 1-D array of the pool's stored elements starting at the view root.
    offsets_row: [2, 4W] P32 indices of this request (row 0 K, row 1 V)."""
    H, d = num_kv_heads, head_dim
    j = np.arange(kv_len, dtype=np.int64)[:, None, None]
    h = np.arange(H, dtype=np.int64)[None, :, None]
    c = np.arange(d, dtype=np.int64)[None, None, :]
    out = []
    for kind in (0, 1):
        x = np.asarray(offsets_row[kind], dtype=np.int64)
        elem = ((x[j // SUB] * H + h) * SUB + j % SUB) * d + c
        out.append(root_flat[elem])
    return out[0], out[1]


def gather_hnd(pool: np.ndarray, block_table_row: np.ndarray, kv_len: int,
               page: int = 128) -> np.ndarray:
    """Logical [kv_len, Hkv, d] of one request from ordinary head-major pages
    [num_pages, Hkv, 128, d]: position j is token j % 128 of page
    block_table_row[j // 128]."""
    n = -(-kv_len // page)
    pages = pool[np.asarray(block_table_row[:n], dtype=np.int64)]   # [n, H, 128, d]
    seq = np.transpose(pages, (0, 2, 1, 3)).reshape(n * page, pool.shape[1], pool.shape[3])
    return seq[:kv_len]


def head_slice_grouped(num_heads: int, h0: int, h1: int, head_dim: int):
    """Descriptors (element offset, length) within one grouped page that cover heads
    [h0, h1): one per 32-token group, in group order."""
    return [((g * num_heads + h0) * SUB * head_dim, (h1 - h0) * SUB * head_dim)
            for g in range(GROUPS)]


def head_slice_contiguous(num_heads: int, h0: int, h1: int, head_dim: int, page: int = 128):
    """The single descriptor of heads [h0, h1) if the page were ordinary
    [heads, 128, d] (the mapping the pages report as wrong for grouped pages)."""
    return [(h0 * page * head_dim, (h1 - h0) * page * head_dim)]


def head_slice_descriptors(token_groups: int, src_heads: int, src_h0: int, dst_heads: int,
                           dst_h0: int, n_heads: int, head_dim: int, elem_bytes: int,
                           src_pages, dst_pages, page_tokens: int = 128):
    """Byte-range copies (src offset, dst offset, length) that move heads
    [src_h0, src_h0 + n_heads) of each source page to heads [dst_h0, dst_h0 + n_heads) of
    the matching destination page.  A page of `token_groups` groups is laid out
    [group, heads, page_tokens / groups, d]; the mapper emits one descriptor per
    (page, token group) — per (layer, K/V, token group) when the page list enumerates
    the layers' K and V pages ([PR17835] item 2).  token_groups = 1 is the ordinary
    head-major slice [heads, page_tokens, d]."""
    tpg = page_tokens // token_groups
    row = tpg * head_dim * elem_bytes            # one head's bytes in one group
    out = []
    for sp, dp in zip(src_pages, dst_pages):
        for g in range(token_groups):
            out.append((int(sp) + (g * src_heads + src_h0) * row,
                        int(dp) + (g * dst_heads + dst_h0) * row, n_heads * row))
    return out


def apply_descriptors(dst_flat: np.ndarray, src_flat: np.ndarray, descriptors) -> None:
    """Copy src sequentially into dst at the descriptor ranges, in order."""
    pos = 0
    for off, length in descriptors:
        dst_flat[off:off + length] = src_flat[pos:pos + length]
        pos += length
    assert pos == src_flat.size
