"""Pins of the oracle's per-tensor fp8 scales in all three attention pipelines (CPU only).

fp8 K/V carry one float32 scale per tensor (value = decode(byte) * scale): K's scale
multiplies every key, V's every value.  The checks below give K and V clearly
different scales (about 0.37x and 2.5x the generated amax/448 ones) and compare each
oracle pipeline with a brute-force loop that addresses the pools directly from the
pages' layout statements and decodes bytes with torch.float8_e4m3fn (a library
routine).  Negative controls show that the comparison would catch the scales
swapped, dropped or applied twice.

Layouts addressed here:
  * dense draft pool: slot s's draft-layer K page is 128-token page s * stride + root
    of the flat pool and its V page the next one; a page is four head-major 32-token
    groups [4][Hkv][32][d], so position j is group (j % 128) // 32, token j % 32
    ([PR18066] view-scale commit; [PR17835] item 2 "Grouped-HND draft KV transfer");
  * head-major pools: position j is token j % 128 of page block_table[r][j // 128],
    [Hkv][128][d] per page ([PR17835] item 2, the ordinary head-major page);
  * token t of a request attends j < kv_len - qo_len + t + 1 ([PR3] MSA verify commit).
"""
import numpy as np
import torch

import oracle
import workloads as W
from workloads import raw_numpy

K_GAIN, V_GAIN = 0.37, 2.5
# bf16 / fp8 tolerance against the float64 truth; every control below must move the
# result by more than this.
TOL = 2e-2

DENSE_FP8 = W.DENSE_BF16.scaled(name="dense_fp8_pin", batch=2, kv=("list", (200, 333)),
                                kv_capacity=384, kv_dtype="fp8", num_q_heads=8, num_kv_heads=2,
                                head_dim=64)
SPARSE_FP8 = W.LONG_FP8.scaled(name="sparse_fp8_pin", batch=2, kv=("list", (300, 517)),
                               kv_capacity=640, num_q_heads=8, num_kv_heads=2, head_dim=64,
                               top_k=2, num_splits=1)


def _fp8_values(raw_u8: np.ndarray) -> np.ndarray:
    """Library decode: the uint8 bytes reinterpreted as torch.float8_e4m3fn, widened."""
    t = torch.from_numpy(np.ascontiguousarray(raw_u8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _softmax_row(q_vec, keys, vals, scale):
    logits = scale * (keys @ q_vec)
    p = np.exp(logits - logits.max())
    return (p[:, None] * vals).sum(0) / p.sum()


def _dense_brute(c, k_scale, v_scale, requests=None):
    w = c.w
    pool = _fp8_values(raw_numpy(c.pool))                  # [slots * stride, 4, Hkv, 32, d]
    q = c.q.to(torch.float64).numpy()                      # library bf16 widening
    ind = c.qo_indptr.numpy()
    bt = c.block_table.numpy()
    G = w.num_q_heads // w.num_kv_heads
    out = np.full(q.shape, np.nan)
    for r in (range(w.batch) if requests is None else requests):
        kv = int(c.lengths.kv[r])
        qo = ind[r + 1] - ind[r]
        j = np.arange(kv)
        kpage = bt[r][j // 128] * w.slot_stride + w.root_page
        grp, tok = (j % 128) // 32, j % 32
        for t in range(qo):
            n = kv - qo + t + 1
            for hq in range(w.num_q_heads):
                h = hq // G
                keys = pool[kpage[:n], grp[:n], h, tok[:n]] * k_scale
                vals = pool[kpage[:n] + 1, grp[:n], h, tok[:n]] * v_scale
                out[ind[r] + t, hq] = _softmax_row(q[ind[r] + t, hq], keys, vals, c.softmax_scale)
    return out


def _headmajor_brute(c, k_scale, v_scale, chosen=None):
    """chosen[row, h] = set of request-local pages token row may see (None: all)."""
    w = c.w
    kp = _fp8_values(raw_numpy(c.k_pool))                  # [pages, Hkv, 128, d]
    vp = _fp8_values(raw_numpy(c.v_pool))
    q = c.q.to(torch.float64).numpy()                      # library bf16 widening
    ind = c.qo_indptr.numpy()
    bt = c.block_table.numpy()
    G = w.num_q_heads // w.num_kv_heads
    out = np.full(q.shape, np.nan)
    for r in range(w.batch):
        kv = int(c.lengths.kv[r])
        qo = ind[r + 1] - ind[r]
        for t in range(qo):
            row = ind[r] + t
            n = kv - qo + t + 1
            for hq in range(w.num_q_heads):
                h = hq // G
                j = np.arange(n)
                if chosen is not None:
                    j = j[np.isin(j // 128, sorted(chosen[row][h]))]
                keys = kp[bt[r][j // 128], h, j % 128] * k_scale
                vals = vp[bt[r][j // 128], h, j % 128] * v_scale
                out[row, hq] = _softmax_row(q[row, hq], keys, vals, c.softmax_scale)
    return out


def _assert_pinned(got, brute_fn, k_scale, v_scale):
    """got matches the brute force at (k_scale, v_scale) and not at the mistaken ones."""
    assert np.allclose(got, brute_fn(k_scale, v_scale), rtol=1e-12, atol=1e-12)
    for name, ks, vs in (("swapped", v_scale, k_scale), ("K dropped", 1.0, v_scale),
                         ("V dropped", k_scale, 1.0), ("K twice", k_scale ** 2, v_scale),
                         ("V twice", k_scale, v_scale ** 2)):
        wrong = brute_fn(ks, vs)
        assert np.nanmax(np.abs(wrong - got)) > TOL, f"{name} scale is not observable"


def _dense_oracle(c, k_scale, v_scale):
    w = c.w
    page_elems = 4 * w.num_kv_heads * 32 * w.head_dim
    return oracle.dense_verify_case(
        raw_numpy(c.q), w.q_dtype, c.qo_indptr.numpy(), c.lengths.kv,
        raw_numpy(c.pool).reshape(-1), w.kv_dtype, w.root_page * page_elems,
        c.block_table.numpy(), w.slot_stride, w.num_kv_heads, w.head_dim, k_scale, v_scale,
        c.softmax_scale)


def _sparse_oracle(c, k_scale, v_scale, top_k):
    w = c.w
    return oracle.sparse_verify_case(
        raw_numpy(c.q), w.q_dtype, c.qo_indptr.numpy(), c.lengths.kv, raw_numpy(c.k_pool),
        raw_numpy(c.v_pool), w.kv_dtype, c.block_table.numpy(), k_scale, v_scale, top_k,
        c.softmax_scale, w.max_pages())


def test_dense_view_pipeline_fp8_distinct_scales():
    c = W.make_dense_case(DENSE_FP8)
    ks, vs = K_GAIN * c.k_scale, V_GAIN * c.v_scale
    got = _dense_oracle(c, ks, vs)
    _assert_pinned(got, lambda a, b: _dense_brute(c, a, b), ks, vs)


def test_dense_view_pipeline_never_reads_poison():
    """Every page other than the draft layer's K/V pages of assigned slots holds NaN: the
    output stays finite and equals the brute force over the pages' addresses."""
    c = W.make_dense_case(DENSE_FP8, poison=True)
    ks, vs = K_GAIN * c.k_scale, V_GAIN * c.v_scale
    got = _dense_oracle(c, ks, vs)
    assert np.all(np.isfinite(got))
    assert np.allclose(got, _dense_brute(c, ks, vs), rtol=1e-12, atol=1e-12)


def test_dense_view_pipeline_fp32_tiny_equals_brute_force():
    c = W.make_dense_case(W.TINY_FP32)
    w = c.w
    page_elems = 4 * w.num_kv_heads * 32 * w.head_dim
    got = oracle.dense_verify_case(
        raw_numpy(c.q), "f32", c.qo_indptr.numpy(), c.lengths.kv, raw_numpy(c.pool).reshape(-1),
        "f32", w.root_page * page_elems, c.block_table.numpy(), w.slot_stride, w.num_kv_heads,
        w.head_dim, 1.0, 1.0, c.softmax_scale)
    pool = raw_numpy(c.pool).astype(np.float64)
    q = raw_numpy(c.q).astype(np.float64)
    ind = c.qo_indptr.numpy()
    bt = c.block_table.numpy()
    G = w.num_q_heads // w.num_kv_heads
    for r in range(w.batch):
        kv, qo = int(c.lengths.kv[r]), ind[r + 1] - ind[r]
        for t in range(qo):
            for hq in range(w.num_q_heads):
                n = kv - qo + t + 1
                keys = np.stack([pool[bt[r][j // 128] * w.slot_stride + w.root_page,
                                      (j % 128) // 32, hq // G, j % 32] for j in range(n)])
                vals = np.stack([pool[bt[r][j // 128] * w.slot_stride + w.root_page + 1,
                                      (j % 128) // 32, hq // G, j % 32] for j in range(n)])
                ref = _softmax_row(q[ind[r] + t, hq], keys, vals, c.softmax_scale)
                assert np.allclose(got[ind[r] + t, hq], ref, rtol=1e-12, atol=1e-12)


def test_sparse_pipeline_fp8_distinct_scales():
    c = W.make_sparse_case(SPARSE_FP8)
    ks, vs = K_GAIN * c.k_scale, V_GAIN * c.v_scale
    res = _sparse_oracle(c, ks, vs, SPARSE_FP8.top_k)
    chosen = [[set(int(p) for p in res["topk"][row, h] if p >= 0)
               for h in range(SPARSE_FP8.num_kv_heads)] for row in range(res["topk"].shape[0])]
    # the selection must be a real subset for some token (the test is about sparse)
    assert any(len(s) < -(-int(c.lengths.kv[1]) // 128) for s in chosen[-1])
    _assert_pinned(res["out"], lambda a, b: _headmajor_brute(c, a, b, chosen), ks, vs)


def test_sparse_scores_ignore_fp8_scales():
    """The proxy scores are unscaled: any K or V scale gives the same scores bit for bit
    and the same selection."""
    c = W.make_sparse_case(SPARSE_FP8)
    a = _sparse_oracle(c, c.k_scale, c.v_scale, SPARSE_FP8.top_k)
    b = _sparse_oracle(c, 7.0 * c.k_scale, 0.1 * c.v_scale, SPARSE_FP8.top_k)
    assert np.array_equal(a["scores"].view(np.uint32), b["scores"].view(np.uint32))
    assert np.array_equal(a["topk"], b["topk"])


def test_paged_pipeline_fp8_distinct_scales():
    c = W.make_sparse_case(SPARSE_FP8)
    ks, vs = K_GAIN * c.k_scale, V_GAIN * c.v_scale
    w = c.w
    got = oracle.paged_verify_case(
        raw_numpy(c.q), w.q_dtype, c.qo_indptr.numpy(), c.lengths.kv, raw_numpy(c.k_pool),
        raw_numpy(c.v_pool), w.kv_dtype, c.block_table.numpy(), ks, vs, c.softmax_scale)
    _assert_pinned(got, lambda a, b: _headmajor_brute(c, a, b), ks, vs)
