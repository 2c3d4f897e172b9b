"""Per-token ladder-bounded top-k page selection.

[PR3] MSA verify commit: top-k selection receives each token's own count of valid
pages under the ladder, so a draft token cannot choose pages past its own attend
bound.  Readings: selection is per (token, KV head); candidates are the pages
p < n_valid(t) = ceil(bound_t / 128); the order is score descending, then page index
ascending (ties go to the lower page); the output lists min(K, n_valid) pages in
that rank order and pads the rest with -1.
"""
import numpy as np

from .ladder import ladder_bounds, n_valid_pages


def ladder_topk_request(scores: np.ndarray, kv_len: int, top_k: int, page: int = 128):
    """scores [qo, Hkv, >= n_pages] -> (idx [qo, Hkv, top_k] int64, cnt [qo, Hkv])."""
    qo, Hkv = scores.shape[:2]
    nv = n_valid_pages(ladder_bounds(kv_len, qo), page)
    idx = np.full((qo, Hkv, top_k), -1, dtype=np.int64)
    cnt = np.zeros((qo, Hkv), dtype=np.int64)
    for t in range(qo):
        n = int(nv[t])
        for h in range(Hkv):
            cand = sorted(range(n), key=lambda p: (-float(scores[t, h, p]), p))
            take = cand[:min(top_k, n)]
            idx[t, h, :len(take)] = take
            cnt[t, h] = len(take)
    return idx, cnt
