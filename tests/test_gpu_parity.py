"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on the
same seeded inputs.  Indices and offsets bit-exact; outputs within tolerance
(fp32: 1e-4 relative + 1e-5; bf16 / fp8 K/V: max-abs 2e-2 against the float64 oracle).
Sizes span several tiles, ragged tails and page-crossing ladders; full-size checks of
the benchmark configuration live in test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_p128_amd as sdv
import workloads as W
from workloads import raw_numpy

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _parity import (DEV, DenseRun, SparseRun, dense_oracle, out_numpy, rows_of,
                         sparse_oracle, tol_ok)

TINY = W.TINY_FP32
DENSE_S = W.DENSE_BF16.scaled(name="dense_small", batch=3, kv=("uniform", 100, 900),
                              kv_capacity=1024)
DENSE_S_FP8 = W.DENSE_BF16.scaled(name="dense_small_fp8", batch=2, kv=("uniform", 33, 700),
                                  kv_capacity=768, kv_dtype="fp8", num_q_heads=16)
RAGGED_S = W.RAGGED_MIXED.scaled(name="ragged_small", batch=24,
                                 kv=("lognormal", 300, 1.0, 1, 2000, 0.25), kv_capacity=2048)
SPARSE_S = W.SPARSE_BF16.scaled(name="sparse_small", batch=3, kv=("uniform", 500, 3000),
                                kv_capacity=3072, top_k=4)
LONG_S = W.LONG_FP8.scaled(name="long_small", batch=2, kv=("fixed", 5000), kv_capacity=5120,
                           top_k=8)
D64 = W.SPARSE_BF16.scaled(name="d64", batch=3, kv=("uniform", 130, 1000), kv_capacity=1024,
                           head_dim=64, num_q_heads=8, num_kv_heads=2, top_k=3)

# eight verify tokens selecting 64 pages each: 512 (token, rank) entries per (request, KV
# head), the most a union takes (two per thread of the workgroup)
WIDE_UNION = W.SPARSE_BF16.scaled(name="wide_union", batch=3, qo=8,
                                  kv=("list", (9000, 12000, 16000)), kv_capacity=16384, top_k=64)

D64_FP8 = W.LONG_FP8.scaled(name="d64_fp8", batch=3, kv=("uniform", 130, 1500), kv_capacity=1536,
                            head_dim=64, num_q_heads=8, num_kv_heads=2, top_k=3)

DENSE_CASES = [TINY, DENSE_S, DENSE_S_FP8, RAGGED_S]
SPARSE_CASES = [TINY, SPARSE_S, LONG_S, RAGGED_S, D64, WIDE_UNION]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


@pytest.mark.parametrize("w", DENSE_CASES, ids=lambda w: w.name)
def test_subpage_offsets_bit_exact(w):
    c = W.make_dense_case(w)
    run = DenseRun(c)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    view, offs = run.view(dev_err=err)
    torch.cuda.synchronize()
    ref = oracle.subpage_offsets(c.block_table.numpy(), w.slot_stride)
    assert np.array_equal(offs.cpu().numpy(), ref.astype(np.int32))
    assert int(err.item()) == 0
    assert view.c.index_scale == w.slot_stride


def test_subpage_offsets_bad_slot_flags_and_maps_to_slot0():
    c = W.make_dense_case(TINY)
    bt = c.block_table.clone()
    bt[1, 0] = c.num_slots + 5
    bt[0, 1] = -1
    run = DenseRun(c)
    run.bt = bt.to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    _, offs = run.view(dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & sdv._lib.DEVERR_PAGE_RANGE
    o = offs.cpu().numpy()
    assert list(o[1, 0, 0:4]) == [0, 1, 2, 3] and list(o[0, 1, 4:8]) == [4, 5, 6, 7]


@pytest.mark.parametrize("family", [0, 1, 3, 4, 5, 6])
@pytest.mark.parametrize("splits", [1, 2, 16])
@pytest.mark.parametrize("w", DENSE_CASES, ids=lambda w: w.name)
def test_dense_parity(w, splits, family):
    c = W.make_dense_case(w)
    run = DenseRun(c)
    view, offs = run.view()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run.attend(view, offs, num_splits=splits, dev_err=err, family=family)
    torch.cuda.synchronize()
    ref = dense_oracle(c)
    ok, worst = tol_ok(out_numpy(out[:run.n]), ref, w.q_dtype if w.kv_dtype != "fp8" else "fp8")
    assert int(err.item()) == 0
    assert ok, f"max abs err {worst}"


# Over 64 requests (two of them a lane in the plan of the dense pieces) and fewer
# (request, KV head) pairs than the GPU holds: the ring kernel's request-sized pieces,
# with unused partial slots marked empty when a pair takes fewer runs than splits.
DENSE_MANY = W.DENSE_BF16.scaled(name="dense_many", batch=100, kv=("uniform", 40, 1200),
                                 kv_capacity=1216)


# Over 128 requests (eight a lane) in fewer than 512 pairs: two KV heads.
DENSE_MANY_200 = W.DENSE_BF16.scaled(name="dense_many_200", batch=200, num_q_heads=16,
                                     num_kv_heads=2, kv=("uniform", 40, 600), kv_capacity=640)


@pytest.fixture(scope="module", params=[DENSE_MANY, DENSE_MANY_200], ids=lambda w: w.name)
def dense_many(request):
    c = W.make_dense_case(request.param)
    return c, dense_oracle(c)


@pytest.mark.parametrize("family", [0, 4])
@pytest.mark.parametrize("splits", [2, 6, 16])
def test_dense_pieces_many_requests(dense_many, splits, family):
    c, ref = dense_many
    run = DenseRun(c)
    view, offs = run.view()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run.attend(view, offs, num_splits=splits, dev_err=err, family=family)
    torch.cuda.synchronize()
    ok, worst = tol_ok(out_numpy(out[:run.n]), ref, "bf16")
    assert int(err.item()) == 0
    assert ok, f"max abs err {worst}"


@pytest.mark.parametrize("w", SPARSE_CASES + [D64_FP8], ids=lambda w: w.name)
def test_proxy_scores_bit_exact(w):
    c = W.make_sparse_case(w)
    run = SparseRun(c)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = run.scores(dev_err=err).cpu().numpy()
    ref = sparse_oracle(c)["scores"]
    ind = c.qo_indptr.numpy()
    for r in range(w.batch):
        n_pages = -(-int(c.lengths.kv[r]) // 128)
        a, b = ind[r], ind[r + 1]
        got = s[a:b, :, :n_pages]
        exp = ref[a:b, :, :n_pages]
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), f"request {r}"
    assert int(err.item()) == 0


@pytest.mark.parametrize("w", SPARSE_CASES, ids=lambda w: w.name)
def test_topk_bit_exact(w):
    c = W.make_sparse_case(w)
    run = SparseRun(c)
    idx, cnt = run.topk(run.scores())
    ref = sparse_oracle(c)
    n = run.n
    assert np.array_equal(idx[:n].cpu().numpy(), ref["topk"][:n].astype(np.int32))
    assert np.array_equal(cnt[:n].cpu().numpy(), ref["count"][:n].astype(np.int32))


def test_topk_integer_ties_from_given_scores():
    # Scores with many exact ties (and -0 vs +0) are fed to both sides.
    rng = np.random.default_rng(0)
    w = W.LONG_FP8.scaled(batch=3, kv=("list", (3000, 129, 9000)), kv_capacity=9216, top_k=64)
    qo, kv = W.draw_lengths(w, 3)
    ind = np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)
    max_pages = w.max_pages()
    rows = int(ind[-1])
    scores = rng.integers(-2, 3, size=(w.batch * w.max_qo(), w.num_kv_heads, max_pages)).astype(np.float32)
    scores[scores == 0] = np.where(rng.random((scores == 0).sum()) < 0.5, -0.0, 0.0)
    idx = sdv.ladder_topk_pages(torch.from_numpy(scores).to(DEV), torch.from_numpy(ind).to(DEV),
                                torch.from_numpy(kv.astype(np.int32)).to(DEV),
                                max_qo_len=w.max_qo(), top_k=w.top_k)
    got = idx.cpu().numpy()
    for r in range(w.batch):
        e, _ = oracle.ladder_topk_request(scores[ind[r]:ind[r + 1]], int(kv[r]), w.top_k)
        assert np.array_equal(got[ind[r]:ind[r + 1]], e.astype(np.int32)), f"request {r}"
    assert rows == w.batch * 4


@pytest.mark.parametrize("family", [0, 1, 3, 4])
@pytest.mark.parametrize("splits", [1, 2, 16])
@pytest.mark.parametrize("w", SPARSE_CASES, ids=lambda w: w.name)
def test_sparse_parity(w, splits, family):
    c = W.make_sparse_case(w)
    run = SparseRun(c)
    idx, _ = run.topk(run.scores())
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run.attend(idx, num_splits=splits, dev_err=err, family=family)
    torch.cuda.synchronize()
    ref = sparse_oracle(c)
    assert np.array_equal(idx[:run.n].cpu().numpy(), ref["topk"][:run.n].astype(np.int32))
    ok, worst = tol_ok(out_numpy(out[:run.n]), ref["out"], "f32" if w.kv_dtype == "f32" else "bf16")
    assert int(err.item()) == 0
    assert ok, f"max abs err {worst}"


RAGGED_MANY = W.RAGGED_MIXED.scaled(name="ragged_many", batch=48,
                                    kv=("lognormal", 300, 1.0, 1, 1500, 0.25), kv_capacity=1536)
RAGGED_MANY_FP8 = RAGGED_MANY.scaled(name="ragged_many_fp8", kv_dtype="fp8")
# 1280 (request, KV head) pairs: more workgroups than the GPU holds even unsplit, so the
# launch takes its requests longest first
RAGGED_ORDER = W.RAGGED_MIXED.scaled(name="ragged_order", batch=320,
                                     kv=("lognormal", 300, 1.0, 1, 1500, 0.25), kv_capacity=1536)


@pytest.mark.parametrize("splits", [1, 4, 8])
@pytest.mark.parametrize("w", [RAGGED_MANY, RAGGED_MANY_FP8, RAGGED_ORDER], ids=lambda w: w.name)
def test_sparse_many_workgroups(w, splits):
    """Ragged 32-row (request, KV head) pairs, bf16 and fp8, in launches of several
    workgroups per CU: the standalone and the fused-selection forms against the oracle,
    and bit-identical to each other."""
    c = W.make_sparse_case(w)
    run = SparseRun(c)
    scores = run.scores()
    idx, _ = run.topk(scores)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run.attend(idx, num_splits=splits, dev_err=err)
    fused = sdv.verify_attention_sparse_select(run.q, run.qo_indptr, run.kv_len, run.kv, run.bt,
                                               scores, max_qo_len=run.max_qo, top_k=w.top_k,
                                               softmax_scale=c.softmax_scale, num_splits=splits,
                                               dev_err=err)
    torch.cuda.synchronize()
    ref = sparse_oracle(c)
    assert int(err.item()) == 0
    ok, worst = tol_ok(out_numpy(out[:run.n]), ref["out"], "bf16")
    assert ok, f"max abs err {worst}"
    assert torch.equal(out[:run.n].view(torch.int16), fused[:run.n].view(torch.int16))


@pytest.mark.parametrize("w", [TINY, SPARSE_S], ids=lambda w: w.name)
def test_sparse_with_every_page_equals_dense(w):
    c = W.make_sparse_case(w)
    run = SparseRun(c)
    K = w.max_pages()
    idx, _ = run.topk(run.scores(), top_k=K)
    out = run.attend(idx)
    torch.cuda.synchronize()
    ind = c.qo_indptr.numpy()
    q = oracle.decode_store(raw_numpy(c.q), w.q_dtype).astype(np.float64)
    got = out_numpy(out[:run.n])
    for r in range(w.batch):
        kvr = int(c.lengths.kv[r])
        k, v = oracle.request_kv_sparse(raw_numpy(c.k_pool), raw_numpy(c.v_pool), w.kv_dtype,
                                        c.block_table[r].numpy(), kvr)
        dense = oracle.dense_verify_request(q[ind[r]:ind[r + 1]], k.astype(np.float64),
                                            v.astype(np.float64), kvr, c.softmax_scale)
        ok, worst = tol_ok(got[ind[r]:ind[r + 1]], dense, "f32" if w.kv_dtype == "f32" else "bf16")
        assert ok, f"request {r}: {worst}"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("S", [1, 3, 4, 7, 16, 23])   # chunks of 4, 8, 16; 23: two chunks
def test_combine_parity(D, out_dtype, S):
    rng = np.random.default_rng(D + 100 * S)
    R, H = 19, 3
    po = rng.standard_normal((S, R, H, D)).astype(np.float32)
    pl = (rng.standard_normal((S, R, H)) * 3).astype(np.float32)
    pl[rng.random((S, R, H)) < 0.3] = -np.inf
    pl[:, 4, 1] = -np.inf                                 # a row with no live partial
    if S > 16:
        pl[:16, 6, 2] = -np.inf                           # live partials only in the second chunk
        pl[16:, 7, 0] = -np.inf                           # ... only in the first
    po[pl == -np.inf] = np.nan                            # never read
    out, lse = sdv.lse_combine(torch.from_numpy(po).to(DEV), torch.from_numpy(pl).to(DEV),
                               out_dtype=out_dtype, want_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.lse_combine(po.reshape(S, R * H, D), pl.reshape(S, R * H))
    ok, worst = tol_ok(out_numpy(out).reshape(R * H, D), ref_o,
                       "f32" if out_dtype == torch.float32 else "bf16")
    assert ok, worst
    gl = lse.cpu().numpy().reshape(-1)
    assert np.array_equal(np.isinf(gl), np.isinf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.allclose(gl[fin], ref_l[fin], rtol=1e-5, atol=1e-5)


def _poison_stale_tail_hnd(pool, bt, kv_lens):
    """NaN in every slot of a request's last page beyond its kv_len (ordinary HND)."""
    for r, kv in enumerate(kv_lens):
        kv = int(kv)
        if kv % 128:
            pool[int(bt[r, kv // 128]), :, kv % 128:, :] = float("nan")


@pytest.mark.parametrize("family", [0, 1, 3, 4])
@pytest.mark.parametrize("w", [SPARSE_S, LONG_S, RAGGED_S], ids=lambda w: w.name)
def test_sparse_poison_never_read(w, family):
    c = W.make_sparse_case(w, poison=True)
    _poison_stale_tail_hnd(c.k_pool, c.block_table, c.lengths.kv)
    _poison_stale_tail_hnd(c.v_pool, c.block_table, c.lengths.kv)
    run = SparseRun(c)
    s = run.scores()
    idx, _ = run.topk(s)
    out = run.attend(idx, num_splits=2, family=family)
    torch.cuda.synchronize()
    ref = sparse_oracle(c)
    assert np.array_equal(idx[:run.n].cpu().numpy(), ref["topk"][:run.n].astype(np.int32))
    ok, worst = tol_ok(out_numpy(out[:run.n]), ref["out"], "bf16")
    assert ok, worst


@pytest.mark.parametrize("family", [0, 1, 3, 4, 5, 6])
def test_dense_poison_never_read(family):
    w = DENSE_S
    c = W.make_dense_case(w, poison=True)
    # NaN in the stale token slots of each request's last page: the page is
    # [4 groups, Hkv, 32, d]; position j is group (j % 128) // 32, token j % 32.
    for r, kv in enumerate(c.lengths.kv):
        kv = int(kv)
        if kv % 128 == 0:
            continue
        slot = int(c.block_table[r, kv // 128])
        for kind in (0, 1):
            page = c.pool[slot * w.slot_stride + w.root_page + kind]
            for j in range(kv % 128, 128):
                page[j // 32, :, j % 32, :] = float("nan")
    run = DenseRun(c)
    view, offs = run.view()
    out = run.attend(view, offs, num_splits=2, family=family)
    torch.cuda.synchronize()
    ok, worst = tol_ok(out_numpy(out[:run.n]), dense_oracle(c), "bf16")
    assert ok, worst


def test_device_error_flags():
    c = W.make_sparse_case(SPARSE_S)
    run = SparseRun(c)
    kv_bad = c.kv_len.clone()
    kv_bad[1] = SPARSE_S.max_pages() * 128 + 1            # beyond the table's capacity
    run.kv_len = kv_bad.to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    run.scores(dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & sdv._lib.DEVERR_KV_CAPACITY
    kv_bad[1] = 2                                         # shorter than qo_len
    run.kv_len = kv_bad.to(DEV)
    err.zero_()
    run.scores(dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & sdv._lib.DEVERR_QO_LEN
    # a top-k entry beyond the token's valid pages
    run.kv_len = c.kv_len.to(DEV)
    idx, _ = run.topk(run.scores())
    idx[0, 0, 0] = 10 ** 6
    err.zero_()
    run.attend(idx, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & sdv._lib.DEVERR_TOPK_INDEX


def test_decode_and_minimum_lengths():
    # qo_len = 1 (ordinary decode), kv_len = qo_len, kv_len a multiple of 128 and
    # kv_len at the table's capacity.
    w = W.SPARSE_BF16.scaled(batch=4, qo=4, kv=("list", (4, 128, 256, 512)), kv_capacity=512,
                             top_k=2)
    for qo in (1, 4):
        wq = w.scaled(qo=qo)
        c = W.make_sparse_case(wq)
        run = SparseRun(c)
        idx, _ = run.topk(run.scores())
        out = run.attend(idx, num_splits=2)
        torch.cuda.synchronize()
        ref = sparse_oracle(c)
        assert np.array_equal(idx[:run.n].cpu().numpy(), ref["topk"][:run.n].astype(np.int32))
        ok, worst = tol_ok(out_numpy(out[:run.n]), ref["out"], "bf16")
        assert ok, worst
        wd = W.DENSE_BF16.scaled(batch=4, qo=qo, kv=("list", (4, 128, 256, 512)), kv_capacity=512)
        d = W.make_dense_case(wd)
        drun = DenseRun(d)
        view, offs = drun.view()
        outd = drun.attend(view, offs, num_splits=3)
        torch.cuda.synchronize()
        ok, worst = tol_ok(out_numpy(outd[:drun.n]), dense_oracle(d), "bf16")
        assert ok, worst


def test_empty_batch_is_a_no_op():
    q = torch.zeros((0, 16, 128), dtype=torch.bfloat16, device=DEV)
    ind = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvl = torch.zeros(0, dtype=torch.int32, device=DEV)
    k = torch.zeros((1, 4, 128, 128), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    kv = sdv.PagedKV(k, k)
    s = sdv.proxy_page_scores(q, ind, kvl, kv, bt, max_qo_len=4)
    assert s.shape[0] == 0


def test_graph_replay_with_mutated_lengths():
    """Capture both paths at short kv_len, then replay after growing the lengths up to
    the table's capacity and shrinking rows across a page boundary (all on device);
    every replay matches the oracle for the lengths it ran with."""
    w = W.SPARSE_BF16.scaled(batch=3, kv=("list", (700, 1500, 2600)), kv_capacity=2688, top_k=4)
    c = W.make_sparse_case(w)
    run = SparseRun(c)
    wd = W.DENSE_BF16.scaled(batch=3, kv=("list", (700, 1500, 2600)), kv_capacity=2688,
                             num_q_heads=16)
    d = W.make_dense_case(wd)
    drun = DenseRun(d)
    view, offs = drun.view()
    kv_dev = torch.tensor([300, 140, 2000], dtype=torch.int32, device=DEV)
    run.kv_len = kv_dev
    drun.kv_len = kv_dev
    rows_cap = w.batch * w.max_qo()
    scores = torch.empty((rows_cap, w.num_kv_heads, w.max_pages()), dtype=torch.float32, device=DEV)
    idx = torch.empty((rows_cap, w.num_kv_heads, w.top_k), dtype=torch.int32, device=DEV)
    cnt = torch.empty((rows_cap, w.num_kv_heads), dtype=torch.int32, device=DEV)
    out = torch.empty((rows_cap, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    outd = torch.empty((rows_cap, wd.num_q_heads, wd.head_dim), dtype=torch.bfloat16, device=DEV)
    ws = sdv.alloc_workspace(rows_cap, w.num_q_heads, w.head_dim, 2, DEV)
    wsd = sdv.alloc_workspace(rows_cap, wd.num_q_heads, wd.head_dim, 3, DEV)

    def path():
        sdv.proxy_page_scores(run.q, run.qo_indptr, kv_dev, run.kv, run.bt, max_qo_len=4,
                              scores=scores)
        sdv.ladder_topk_pages(scores, run.qo_indptr, kv_dev, max_qo_len=4, top_k=w.top_k,
                              topk_idx=idx, topk_cnt=cnt)
        sdv.verify_attention_sparse(run.q, run.qo_indptr, kv_dev, run.kv, run.bt, idx,
                                    max_qo_len=4, softmax_scale=c.softmax_scale, num_splits=2,
                                    workspace=ws, out=out)
        sdv.verify_attention_dense(drun.q, drun.qo_indptr, kv_dev, view, offs, max_qo_len=4,
                                   softmax_scale=d.softmax_scale, num_splits=3, workspace=wsd,
                                   out=outd)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        path()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    torch.cuda.synchronize()

    for kvs in ([300, 140, 2000], [700, 1500, 2600], [700, 128, 2560], [129, 1500, 2688],
                [700, 1500, 2600]):
        kv_dev.copy_(torch.tensor(kvs, dtype=torch.int32))
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=DEV) * 2          # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        del junk
        ref = oracle.sparse_verify_case(raw_numpy(c.q), "bf16", c.qo_indptr.numpy(), np.array(kvs),
                                        raw_numpy(c.k_pool), raw_numpy(c.v_pool), "bf16",
                                        c.block_table.numpy(), 1.0, 1.0, w.top_k,
                                        c.softmax_scale, w.max_pages())
        n = run.n
        assert np.array_equal(idx[:n].cpu().numpy(), ref["topk"][:n].astype(np.int32)), kvs
        ok, worst = tol_ok(out_numpy(out[:n]), ref["out"], "bf16")
        assert ok, (kvs, worst)
        dd = W.DenseCase(**{**d.__dict__})
        dd.lengths = W.Lengths(d.lengths.qo, np.array(kvs))
        ok, worst = tol_ok(out_numpy(outd[:n]), dense_oracle(dd), "bf16")
        assert ok, (kvs, worst)
