"""Proxy page scores of the block-sparse target layer.

[PR3] MSA verify commit: the proxy ("OnlyScore") pass runs natively multi-token,
scoring every KV page for every verify token in one pass, under the inclusive causal
bound with offset kv_len - qo_len, i.e. token t sees kv_len - qo_len + t + 1
positions.  The pages name the pass but do not give its formula.

Definition used (a reading, fixed for this library):
  score(t, h, p) = max over query heads hq of KV head h of  q[t, hq] . ksum(t, h, p)
  ksum(t, h, p)  = sum of K[j, h, :] over positions j of page p with j < bound_t
  score = -inf for pages p >= ceil(bound_t / 128) (no attended position).
Unscaled (no 1/sqrt(d), no fp8 scale: a positive constant does not change the
ranking).  The fixed float32 evaluation order that makes the result reproducible
bit for bit:
  1. ksum[c] = (((0 + k_first[c]) + k_next[c]) + ...), positions ascending;
  2. u[c] = q[c] * ksum[c], each product rounded to float32 (no fused multiply-add);
  3. recursive halving over channels: for n = d, d/2, ..., 2: u[c] += u[c + n/2]
     for c < n/2; the dot product is u[0];
  4. maximum over the G query heads; a negative zero becomes +0.
"""
import numpy as np

from .ladder import ladder_bounds, n_valid_pages

PAGE = 128


def canonical_dot_f32(q: np.ndarray, ksum: np.ndarray) -> np.ndarray:
    """Steps 2-3 on the last axis (length d, a power of two); float32 throughout."""
    u = (np.asarray(q, dtype=np.float32) * np.asarray(ksum, dtype=np.float32)).astype(np.float32)
    n = u.shape[-1]
    assert n & (n - 1) == 0, "head_dim must be a power of two"
    while n > 1:
        half = n // 2
        u = (u[..., :half] + u[..., half:n]).astype(np.float32)
        n = half
    return u[..., 0]


def page_prefix_sums_f32(k_seq_h: np.ndarray, n_pages: int, page: int = PAGE) -> np.ndarray:
    """Step 1 for every prefix length: out[p, L, :] = ordered float32 sum of the first
    L keys of page p (L = 0..128).  Sequential accumulation (np.add.accumulate is a
    running sum, unlike np.sum's pairwise reduction)."""
    kv, d = k_seq_h.shape
    padded = np.zeros((n_pages * page, d), dtype=np.float32)
    padded[:kv] = k_seq_h
    pages = padded.reshape(n_pages, page, d)
    with_zero = np.concatenate([np.zeros((n_pages, 1, d), dtype=np.float32), pages], axis=1)
    return np.add.accumulate(with_zero, axis=1, dtype=np.float32)


def proxy_scores_request(q_req: np.ndarray, k_seq: np.ndarray, kv_len: int,
                         page: int = PAGE, heads=None) -> np.ndarray:
    """Scores [qo, Hkv, n_pages] float32 for one request.

    q_req [qo, Hq, d] float32 values; k_seq [kv_len, Hkv, d] float32 values (decoded,
    unscaled).  n_pages = ceil(kv_len / 128).  `heads` restricts the KV heads scored
    (others stay NaN) to bound the cost of sampled checks."""
    qo, Hq, d = q_req.shape
    Hkv = k_seq.shape[1]
    G = Hq // Hkv
    bound = ladder_bounds(kv_len, qo)
    n_pages = int(n_valid_pages(kv_len, page))
    p = np.arange(n_pages)
    out = np.full((qo, Hkv, n_pages), np.nan, dtype=np.float32)
    for h in (range(Hkv) if heads is None else heads):
        pref = page_prefix_sums_f32(np.asarray(k_seq[:, h, :], dtype=np.float32), n_pages, page)
        for t in range(qo):
            L = np.clip(bound[t] - page * p, 0, page)                    # [n_pages]
            ksum = pref[p, L, :]                                        # [n_pages, d]
            best = np.full(n_pages, -np.inf, dtype=np.float32)
            for g in range(G):
                s = canonical_dot_f32(q_req[t, h * G + g, :][None, :], ksum)
                best = np.maximum(best, s)
            best = (best + np.float32(0.0)).astype(np.float32)         # -0 -> +0
            best[L == 0] = -np.inf
            out[t, h, :] = best
    return out
