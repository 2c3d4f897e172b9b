"""Pins for the oracle's verify attention and split-KV combine (CPU only).

Library routine: torch.nn.functional.scaled_dot_product_attention on the CPU in
float64 with an explicit boolean mask built here from the ladder's closed form.
Identities from the pages ([PR3] MSA verify commit): the ladder mask equals the old
single-token math at qo_len = 1, and each verify token equals a single-token
pseudo-row that keeps the request's pages with the ladder as a per-row offset.
"""
import itertools
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def _rand_req(rng, qo, Hq, Hkv, d, kv):
    q = rng.standard_normal((qo, Hq, d))
    k = rng.standard_normal((kv, Hkv, d))
    v = rng.standard_normal((kv, Hkv, d))
    return q, k, v


def _sdpa(q, k, v, allowed_t, G, scale):
    """q [qo, Hq, d], k/v [kv, Hkv, d], allowed_t [qo, kv] (per token, all heads)."""
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq, qo, d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
    mask = torch.from_numpy(allowed_t)[None].expand(qt.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("qo,kv,Hq,Hkv,d", [(4, 300, 8, 2, 64), (1, 17, 4, 4, 8), (8, 9, 16, 4, 16),
                                            (4, 4, 4, 1, 32), (3, 129, 6, 3, 8)])
def test_dense_matches_torch_sdpa(qo, kv, Hq, Hkv, d):
    rng = np.random.default_rng(qo * 1000 + kv)
    q, k, v = _rand_req(rng, qo, Hq, Hkv, d, kv)
    scale = 1.0 / math.sqrt(d)
    bound = kv - qo + np.arange(qo) + 1                            # closed form, written here
    allowed = np.arange(kv)[None, :] < bound[:, None]
    ref = _sdpa(q, k, v, allowed, Hq // Hkv, scale)
    out = oracle.dense_verify_request(q, k, v, kv, scale)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_dense_brute_force_tiny():
    rng = np.random.default_rng(5)
    qo, kv, d = 2, 5, 3
    q, k, v = _rand_req(rng, qo, 2, 1, d, kv)
    out = oracle.dense_verify_request(q, k, v, kv, 0.7)
    for t, hq in itertools.product(range(qo), range(2)):
        n = kv - qo + t + 1
        w = [math.exp(0.7 * sum(q[t, hq, c] * k[j, 0, c] for c in range(d))) for j in range(n)]
        z = sum(w)
        for c in range(d):
            assert abs(out[t, hq, c] - sum(w[j] * v[j, 0, c] for j in range(n)) / z) < 1e-12


def test_row_expansion_identity_dense():
    # Token t of a multi-token request equals a qo_len = 1 request whose kv_len is
    # the token's bound.
    rng = np.random.default_rng(11)
    qo, kv, Hq, Hkv, d = 5, 200, 8, 2, 16
    q, k, v = _rand_req(rng, qo, Hq, Hkv, d, kv)
    out = oracle.dense_verify_request(q, k, v, kv, 0.25)
    for t in range(qo):
        b = kv - qo + t + 1
        single = oracle.dense_verify_request(q[t:t + 1], k[:b], v[:b], b, 0.25)
        assert np.allclose(out[t], single[0], rtol=1e-13, atol=1e-13)


def test_constant_values_give_the_constant():
    rng = np.random.default_rng(2)
    q, k, _ = _rand_req(rng, 4, 4, 2, 8, 50)
    v = np.full((50, 2, 8), 3.25)
    out = oracle.dense_verify_request(q, k, v, 50, 0.3)
    assert np.allclose(out, 3.25, rtol=0, atol=1e-13)


def _page_sets(rng, qo, Hkv, kv, K):
    nv = -(-(kv - qo + np.arange(qo) + 1) // 128)
    idx = np.full((qo, Hkv, K), -1)
    for t in range(qo):
        for h in range(Hkv):
            sel = rng.permutation(int(nv[t]))[:min(K, int(nv[t]))]
            idx[t, h, :len(sel)] = sel
    return idx


@pytest.mark.parametrize("qo,kv,K", [(4, 517, 2), (4, 300, 1), (1, 1000, 3), (7, 1030, 4)])
def test_sparse_matches_masked_sdpa(qo, kv, K):
    rng = np.random.default_rng(kv + K)
    Hq, Hkv, d = 8, 2, 16
    q, k, v = _rand_req(rng, qo, Hq, Hkv, d, kv)
    idx = _page_sets(rng, qo, Hkv, kv, K)
    out = oracle.sparse_verify_request(q, k, v, kv, idx, 0.25)
    G = Hq // Hkv
    for h in range(Hkv):
        allowed = np.zeros((qo, kv), dtype=bool)
        for t in range(qo):
            for p in idx[t, h]:
                if p >= 0:
                    lo, hi = 128 * p, min(128 * (p + 1), kv - qo + t + 1)
                    allowed[t, lo:hi] = True
        ref = _sdpa(q[:, h * G:(h + 1) * G], k[:, h:h + 1], v[:, h:h + 1], allowed, G, 0.25)
        assert np.allclose(out[:, h * G:(h + 1) * G], ref, rtol=1e-12, atol=1e-12)


def test_sparse_with_every_page_equals_dense():
    rng = np.random.default_rng(9)
    qo, kv, Hq, Hkv, d = 4, 777, 8, 2, 16
    q, k, v = _rand_req(rng, qo, Hq, Hkv, d, kv)
    n = -(-kv // 128)
    idx = np.tile(np.arange(n + 3) - 0, (qo, Hkv, 1))
    idx[idx >= n] = -1
    assert np.allclose(oracle.sparse_verify_request(q, k, v, kv, idx, 0.2),
                       oracle.dense_verify_request(q, k, v, kv, 0.2), rtol=1e-13, atol=1e-13)


def test_sparse_row_expansion_identity():
    # [PR3]: the sparse pass row-expands each token to a qo_len = 1 pseudo-row with
    # the request's full page table and the ladder as a per-row offset.
    rng = np.random.default_rng(13)
    qo, kv, Hq, Hkv, d, K = 4, 640, 4, 2, 8, 2
    q, k, v = _rand_req(rng, qo, Hq, Hkv, d, kv)
    idx = _page_sets(rng, qo, Hkv, kv, K)
    out = oracle.sparse_verify_request(q, k, v, kv, idx, 0.3)
    for t in range(qo):
        b = kv - qo + t + 1
        single = oracle.sparse_verify_request(q[t:t + 1], k[:b], v[:b], b, idx[t:t + 1], 0.3)
        assert np.allclose(out[t], single[0], rtol=1e-13, atol=1e-13)


def test_attend_lse_is_logsumexp():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 8))
    k = rng.standard_normal((20, 8))
    v = rng.standard_normal((20, 8))
    allowed = rng.random((3, 20)) < 0.6
    allowed[2] = False
    out, lse = oracle.attend(q, k, v, allowed, 0.5)
    for r in range(2):
        s = 0.5 * (q[r] @ k.T)[allowed[r]]
        assert abs(lse[r] - logsumexp(s)) < 1e-12
    assert lse[2] == -np.inf and np.all(out[2] == 0)


def test_split_combine_equals_whole():
    rng = np.random.default_rng(21)
    R, n, d = 6, 300, 16
    q = rng.standard_normal((R, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    allowed = np.arange(n)[None, :] < rng.integers(1, n, size=R)[:, None]
    whole, whole_lse = oracle.attend(q, k, v, allowed, 0.3)
    for S in (1, 2, 16, 40):
        cuts = np.linspace(0, n, S + 1).astype(int)
        po, pl = [], []
        for s in range(S):
            m = np.zeros_like(allowed)
            m[:, cuts[s]:cuts[s + 1]] = allowed[:, cuts[s]:cuts[s + 1]]
            o, l = oracle.attend(q, k, v, m, 0.3)
            po.append(o)
            pl.append(l)
        out, lse = oracle.lse_combine(np.stack(po), np.stack(pl))
        assert np.allclose(out, whole, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse, whole_lse, rtol=1e-12, atol=1e-12)


def test_combine_all_empty_row():
    out, lse = oracle.lse_combine(np.full((3, 1, 4), np.nan), np.full((3, 1), -np.inf))
    assert lse[0] == -np.inf and np.all(out == 0)


def test_poisoned_unused_values_do_not_leak():
    # A key/value column no row may see must not reach any output, even as NaN;
    # a NaN a row may see must reach it.
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 4))
    k = rng.standard_normal((10, 4))
    v = rng.standard_normal((10, 4))
    allowed = np.ones((3, 10), dtype=bool)
    allowed[:, 7] = False
    k[7] = np.nan
    v[7] = np.nan
    out, lse = oracle.attend(q, k, v, allowed, 0.5)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    allowed[1, 7] = True
    out, _ = oracle.attend(q, k, v, allowed, 0.5)
    assert np.all(np.isnan(out[1])) and np.all(np.isfinite(out[[0, 2]]))
