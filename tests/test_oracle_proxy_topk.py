"""Pins for the oracle's proxy page scores and ladder top-k (CPU only).

On integer data every partial sum is an integer below 2^24, so float32 is exact and
the scores must equal Python-integer brute force regardless of order.  On float
data the evaluation order is a definition; it is pinned by hand-expanded
expressions and by showing that the order is observable.
"""
import numpy as np
import pytest

import oracle
from oracle.proxy import page_prefix_sums_f32


def _brute_scores(q, k, kv, page=128):
    """Python integers: max over the group of sum_{j in page, j < bound} q . k_j."""
    qo, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    n_pages = -(-kv // page)
    out = np.full((qo, Hkv, n_pages), -np.inf)
    for t in range(qo):
        bound = kv - qo + t + 1
        for h in range(Hkv):
            for p in range(n_pages):
                pos = [j for j in range(page * p, page * (p + 1)) if j < bound]
                if not pos:
                    continue
                best = None
                for g in range(G):
                    s = sum(int(q[t, h * G + g, c]) * int(k[j, h, c]) for j in pos for c in range(d))
                    best = s if best is None else max(best, s)
                out[t, h, p] = best
    return out


@pytest.mark.parametrize("qo,kv,d", [(4, 300, 8), (4, 517, 4), (1, 128, 4), (3, 130, 8), (8, 257, 4)])
def test_integer_scores_exact(qo, kv, d):
    rng = np.random.default_rng(kv * 10 + qo)
    Hq, Hkv = 4, 2
    q = rng.integers(-4, 5, size=(qo, Hq, d)).astype(np.float32)
    k = rng.integers(-4, 5, size=(kv, Hkv, d)).astype(np.float32)
    got = oracle.proxy_scores_request(q, k, kv)
    ref = _brute_scores(q, k, kv)
    assert np.array_equal(got, ref.astype(np.float32))


def test_accumulate_is_sequential():
    # The oracle's per-channel key sum runs left to right; on this data the
    # sequential and pairwise orders give different float32 results.
    k = np.zeros((128, 1), dtype=np.float32)
    k[0] = 1.0
    k[1:, 0] = 2.0 ** -24
    pref = page_prefix_sums_f32(k, 1)
    seq = np.float32(0.0)
    for x in k[:, 0]:
        seq = np.float32(seq + x)
    assert pref[0, 128, 0] == seq == np.float32(1.0)            # each tiny add rounds away
    assert np.float32(k[:, 0].sum(dtype=np.float32)) != seq    # numpy's pairwise sum differs


def test_canonical_dot_order_by_hand():
    rng = np.random.default_rng(0)
    f = np.float32
    for _ in range(200):
        q = rng.standard_normal(8).astype(np.float32) * f(1e3)
        k = rng.standard_normal(8).astype(np.float32)
        u = [f(q[c] * k[c]) for c in range(8)]
        by_hand = f(f(f(u[0] + u[4]) + f(u[2] + u[6])) + f(f(u[1] + u[5]) + f(u[3] + u[7])))
        assert oracle.canonical_dot_f32(q, k) == by_hand
        q4, k4 = q[:4], k[:4]
        u4 = [f(q4[c] * k4[c]) for c in range(4)]
        assert oracle.canonical_dot_f32(q4, k4) == f(f(u4[0] + u4[2]) + f(u4[1] + u4[3]))


def test_scores_close_to_float64_and_invalid_pages():
    rng = np.random.default_rng(3)
    qo, kv, Hq, Hkv, d = 4, 390, 8, 2, 32
    q = rng.standard_normal((qo, Hq, d)).astype(np.float32)
    k = rng.standard_normal((kv, Hkv, d)).astype(np.float32)
    s = oracle.proxy_scores_request(q, k, kv)
    G = Hq // Hkv
    for t in range(qo):
        bound = kv - qo + t + 1
        for h in range(Hkv):
            for p in range(s.shape[2]):
                lo, hi = 128 * p, min(128 * (p + 1), bound)
                if lo >= bound:
                    assert s[t, h, p] == -np.inf
                    continue
                ks = k[lo:hi, h, :].astype(np.float64).sum(axis=0)
                ref = max(float(q[t, h * G + g].astype(np.float64) @ ks) for g in range(G))
                assert abs(s[t, h, p] - ref) <= 1e-5 * (1 + abs(ref))


def test_negative_zero_canonical():
    q = np.zeros((1, 1, 4), dtype=np.float32)
    q[0, 0, 0] = -1.0
    k = np.zeros((1, 1, 4), dtype=np.float32)
    s = oracle.proxy_scores_request(q, k, 1)
    assert s[0, 0, 0] == 0 and not np.signbit(s[0, 0, 0])


def _argmax_selection(scores_row, n, K):
    """Independent of sorting: repeatedly take the best remaining page (first max)."""
    left = list(range(n))
    out = []
    while left and len(out) < K:
        best = left[0]
        for p in left[1:]:
            if scores_row[p] > scores_row[best]:
                best = p
        out.append(best)
        left.remove(best)
    return out


@pytest.mark.parametrize("qo,kv,K", [(4, 300, 2), (4, 517, 2), (8, 1030, 3), (1, 64, 5), (4, 2000, 64)])
def test_topk_brute_force_with_ties(qo, kv, K):
    rng = np.random.default_rng(kv + K)
    n_pages = -(-kv // 128)
    scores = rng.integers(-3, 4, size=(qo, 2, n_pages)).astype(np.float32)   # many ties
    idx, cnt = oracle.ladder_topk_request(scores, kv, K)
    for t in range(qo):
        n = -(-(kv - qo + t + 1) // 128)
        for h in range(2):
            ref = _argmax_selection(scores[t, h], n, K)
            assert list(idx[t, h, :len(ref)]) == ref
            assert np.all(idx[t, h, len(ref):] == -1)
            assert cnt[t, h] == min(K, n)
            sel = idx[t, h, :cnt[t, h]]
            assert len(set(sel.tolist())) == len(sel) and np.all(sel < n)
            assert np.all(np.diff(scores[t, h, sel]) <= 0)


def test_topk_ladder_bound_excludes_later_pages():
    # A draft token must not select pages past its own bound even if they score higher.
    kv, qo = 257, 4                     # bounds 254..257: tokens 0-2 see 2 pages, token 3 sees 3
    scores = np.zeros((qo, 1, 3), dtype=np.float32)
    scores[:, 0, 2] = 100.0
    idx, cnt = oracle.ladder_topk_request(scores, kv, 1)
    assert list(idx[:, 0, 0]) == [0, 0, 0, 2]
    assert list(cnt[:, 0]) == [1, 1, 1, 1]
