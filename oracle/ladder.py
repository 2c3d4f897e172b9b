"""The verify ladder.

[PR3] MSA verify commit: with offset = kv_len - qo_len, the inclusive causal bound
makes token t (0 <= t < qo_len) of a request attend kv_len - qo_len + t + 1
positions, kv_len counting the request's own qo_len verify tokens.  Top-k page
selection is bounded by each token's own number of valid pages.
"""
import numpy as np

PAGE = 128


def ladder_bounds(kv_len: int, qo_len: int) -> np.ndarray:
    """Positions each verify token attends: bound[t] = kv_len - qo_len + t + 1."""
    kv_len, qo_len = int(kv_len), int(qo_len)
    if not (1 <= qo_len <= kv_len):
        raise ValueError(f"need 1 <= qo_len ({qo_len}) <= kv_len ({kv_len})")
    return np.arange(qo_len, dtype=np.int64) + (kv_len - qo_len + 1)


def n_valid_pages(bound, page: int = PAGE):
    """Pages holding at least one attended position: ceil(bound / page)."""
    return -(-np.asarray(bound, dtype=np.int64) // page)
