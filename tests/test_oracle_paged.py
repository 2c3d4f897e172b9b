"""Pins of the oracle's dense verify over ordinary head-major P128 pages (the target's
dense layers with the ladder mask): it must equal the sparse oracle when every valid
page is selected, and a brute-force loop that addresses the pools directly."""
import numpy as np

import oracle
import workloads as W
from workloads import raw_numpy

SMALL_BF16 = W.SPARSE_BF16.scaled(name="paged_small", batch=3, kv=("uniform", 130, 700),
                                  kv_capacity=768, top_k=6)


def _paged(c, requests=None):
    w = c.w
    return oracle.paged_verify_case(
        raw_numpy(c.q), w.q_dtype, c.qo_indptr.numpy(), c.lengths.kv, raw_numpy(c.k_pool),
        raw_numpy(c.v_pool), w.kv_dtype, c.block_table.numpy(), c.k_scale, c.v_scale,
        c.softmax_scale, requests=requests)


def test_paged_equals_sparse_with_every_page_selected():
    for w in (W.TINY_FP32, SMALL_BF16):
        c = W.make_sparse_case(w)
        n_pages = int(-(-c.lengths.kv.max() // 128))
        ref = oracle.sparse_verify_case(
            raw_numpy(c.q), w.q_dtype, c.qo_indptr.numpy(), c.lengths.kv, raw_numpy(c.k_pool),
            raw_numpy(c.v_pool), w.kv_dtype, c.block_table.numpy(), c.k_scale, c.v_scale,
            n_pages, c.softmax_scale, w.max_pages())["out"]
        got = _paged(c)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_paged_equals_direct_pool_addressing_brute_force():
    """Position j of request r is token j % 128 of page block_table[r][j // 128]; token t
    attends j < kv_len - qo_len + t + 1; query head hq reads KV head hq // G."""
    c = W.make_sparse_case(W.TINY_FP32)
    w = c.w
    q = raw_numpy(c.q).astype(np.float64)
    kp = raw_numpy(c.k_pool).astype(np.float64) * c.k_scale
    vp = raw_numpy(c.v_pool).astype(np.float64) * c.v_scale
    bt = c.block_table.numpy()
    ind = c.qo_indptr.numpy()
    G = w.num_q_heads // w.num_kv_heads
    got = _paged(c)
    for r in range(w.batch):
        qo = ind[r + 1] - ind[r]
        kv = int(c.lengths.kv[r])
        for t in range(qo):
            bound = kv - qo + t + 1
            for hq in range(w.num_q_heads):
                h = hq // G
                logits, vals = [], []
                for j in range(bound):
                    page, slot = bt[r][j // 128], j % 128
                    logits.append(c.softmax_scale * float(q[ind[r] + t, hq] @ kp[page, h, slot]))
                    vals.append(vp[page, h, slot])
                logits = np.array(logits)
                p = np.exp(logits - logits.max())
                ref = (p[:, None] * np.array(vals)).sum(0) / p.sum()
                assert np.allclose(got[ind[r] + t, hq], ref, rtol=1e-12, atol=1e-12)


def test_paged_rows_outside_sample_stay_nan():
    c = W.make_sparse_case(SMALL_BF16)
    got = _paged(c, requests=[1])
    ind = c.qo_indptr.numpy()
    assert np.isnan(got[: ind[1]]).all() and np.isfinite(got[ind[1]: ind[2]]).all()
