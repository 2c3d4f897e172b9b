"""GPU parity of verify_attention_sparse_select: the per-token ladder top-k taken inside
the sparse attention launch.  The selection it writes out is compared bit-exact with
the oracle's ladder top-k, the output within tolerance with the oracle, and bit-exact
with the two-launch path (standalone top-k, then sparse attention over its indices)
of the same kernel family, which reads the same pages in the same order."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_p128_amd as sdv
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _parity import DEV, SparseRun, out_numpy, sparse_oracle, tol_ok

TINY = W.TINY_FP32
SPARSE_S = W.SPARSE_BF16.scaled(name="sparse_small", batch=3, kv=("uniform", 500, 3000),
                                kv_capacity=3072, top_k=4)
LONG_S = W.LONG_FP8.scaled(name="long_small", batch=2, kv=("fixed", 5000), kv_capacity=5120,
                           top_k=8)
RAGGED_S = W.RAGGED_MIXED.scaled(name="ragged_small", batch=24,
                                 kv=("lognormal", 300, 1.0, 1, 2000, 0.25), kv_capacity=2048)
D64 = W.SPARSE_BF16.scaled(name="d64", batch=3, kv=("uniform", 130, 1000), kv_capacity=1024,
                           head_dim=64, num_q_heads=8, num_kv_heads=2, top_k=3)
# selection over the largest page count the in-kernel top-k takes (1024 pages)
WIDE = W.LONG_FP8.scaled(name="wide_1024_pages", batch=2, kv=("list", (131072, 70001)),
                         kv_capacity=131072, top_k=16, num_q_heads=8, num_kv_heads=1)
# top-64 over up to 1024 pages: tokens with 11 or more key slots a lane (over 640 valid
# pages) select by the bit search inside the attention kernel, the 547-page request by
# the repeated maximum
WIDE_K64 = W.LONG_FP8.scaled(name="wide_top64", batch=3, kv=("list", (131072, 100001, 70001)),
                             kv_capacity=131072, top_k=64, num_q_heads=8, num_kv_heads=1)
# eight tokens selecting 64 pages each: the union's 512-entry limit
WIDE_UNION = W.SPARSE_BF16.scaled(name="wide_union", batch=3, qo=8,
                                  kv=("list", (9000, 12000, 16000)), kv_capacity=16384, top_k=64)
CASES = [TINY, SPARSE_S, LONG_S, RAGGED_S, D64, WIDE_UNION]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


def _select(run, scores, num_splits, write=True, dev_err=None, top_k=None, family=0):
    w = run.c.w
    k = top_k or w.top_k
    rows_cap = w.batch * w.max_qo()
    idx = cnt = None
    if write:
        idx = torch.full((rows_cap, w.num_kv_heads, k), -7, dtype=torch.int32, device=DEV)
        cnt = torch.full((rows_cap, w.num_kv_heads), -7, dtype=torch.int32, device=DEV)
    out = sdv.verify_attention_sparse_select(
        run.q, run.qo_indptr, run.kv_len, run.kv, run.bt, scores, max_qo_len=run.max_qo,
        top_k=k, softmax_scale=run.c.softmax_scale, num_splits=num_splits, topk_idx=idx,
        topk_cnt=cnt, dev_err=dev_err, family=family)
    return out, idx, cnt


@pytest.mark.parametrize("family", [0, 1, 3, 4])
@pytest.mark.parametrize("splits", [1, 2, 16])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_select_parity(w, splits, family):
    c = W.make_sparse_case(w)
    run = SparseRun(c)
    scores = run.scores()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, idx, cnt = _select(run, scores, splits, dev_err=err, family=family)
    idx2, _ = run.topk(scores)
    out2 = run.attend(idx2, num_splits=splits, family=family)
    torch.cuda.synchronize()
    ref = sparse_oracle(c)
    n = run.n
    assert np.array_equal(idx[:n].cpu().numpy(), ref["topk"][:n].astype(np.int32))
    assert np.array_equal(cnt[:n].cpu().numpy(), ref["count"][:n].astype(np.int32))
    ok, worst = tol_ok(out_numpy(out[:n]), ref["out"], "f32" if w.kv_dtype == "f32" else "bf16")
    assert int(err.item()) == 0
    assert ok, f"max abs err {worst}"
    assert torch.equal(out[:n], out2[:n]), "fused and two-launch outputs differ"


@pytest.mark.parametrize("family", [0, 3, 4])
def test_select_without_writing_the_selection(family):
    c = W.make_sparse_case(SPARSE_S)
    run = SparseRun(c)
    out, _, _ = _select(run, run.scores(), 2, write=False, family=family)
    torch.cuda.synchronize()
    ok, worst = tol_ok(out_numpy(out[:run.n]), sparse_oracle(c)["out"], "bf16")
    assert ok, worst


def test_select_widest_table():
    c = W.make_sparse_case(WIDE)
    run = SparseRun(c)
    assert run.bt.shape[1] == 1024
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, idx, cnt = _select(run, run.scores(), 4, dev_err=err)
    torch.cuda.synchronize()
    ref = sparse_oracle(c)
    n = run.n
    assert np.array_equal(idx[:n].cpu().numpy(), ref["topk"][:n].astype(np.int32))
    assert np.array_equal(cnt[:n].cpu().numpy(), ref["count"][:n].astype(np.int32))
    ok, worst = tol_ok(out_numpy(out[:n]), ref["out"], "bf16")
    assert int(err.item()) == 0
    assert ok, worst


@pytest.mark.parametrize("splits", [1, 16])
def test_select_bit_search_top64(splits):
    c = W.make_sparse_case(WIDE_K64)
    run = SparseRun(c)
    scores = run.scores()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, idx, cnt = _select(run, scores, splits, dev_err=err)
    idx2, _ = run.topk(scores)
    out2 = run.attend(idx2, num_splits=splits)
    torch.cuda.synchronize()
    ref = sparse_oracle(c)
    n = run.n
    assert np.array_equal(idx[:n].cpu().numpy(), ref["topk"][:n].astype(np.int32))
    assert np.array_equal(cnt[:n].cpu().numpy(), ref["count"][:n].astype(np.int32))
    ok, worst = tol_ok(out_numpy(out[:n]), ref["out"], "bf16")
    assert int(err.item()) == 0
    assert ok, worst
    assert torch.equal(out[:n], out2[:n]), "fused and two-launch outputs differ"


def test_select_bit_search_ties_and_signed_zeros():
    # six score values (with -0 and +0) over 1024 pages: the k-th largest key sits inside
    # long runs of equal scores, which the page word must order
    c = W.make_sparse_case(WIDE_K64)
    run = SparseRun(c)
    w = WIDE_K64
    rng = np.random.default_rng(11)
    vals = np.array([-2.0, -0.0, 0.0, 0.25, 1.0, 3.0], dtype=np.float32)
    s_np = vals[rng.integers(0, len(vals), size=(w.batch * w.max_qo(), w.num_kv_heads,
                                                   w.max_pages()))]
    scores = torch.from_numpy(s_np).to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, idx, cnt = _select(run, scores, 4, dev_err=err)
    idx2, _ = run.topk(scores)
    out2 = run.attend(idx2, num_splits=4)
    torch.cuda.synchronize()
    got, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    ind = c.qo_indptr.numpy()
    for r in range(w.batch):
        a, b = ind[r], ind[r + 1]
        e, ec = oracle.ladder_topk_request(s_np[a:b], int(c.lengths.kv[r]), w.top_k)
        assert np.array_equal(got[a:b], e.astype(np.int32)), f"request {r}"
        assert np.array_equal(gcnt[a:b], ec.astype(np.int32)), f"request {r}"
    assert int(err.item()) == 0
    assert torch.equal(out[:run.n], out2[:run.n]), "fused and two-launch outputs differ"


@pytest.mark.parametrize("splits", [1, 2])
@pytest.mark.parametrize("w", [SPARSE_S, RAGGED_S], ids=lambda w: w.name)
def test_select_union_only_ties(w, splits):
    # six score values (with -0 and +0) over tables of up to a few hundred pages: the
    # selection that only feeds the page union (no ranked output asked for) must take the
    # same pages as the standalone top-k, ties going to the lower page
    c = W.make_sparse_case(w)
    run = SparseRun(c)
    rng = np.random.default_rng(12)
    vals = np.array([-2.0, -0.0, 0.0, 0.25, 1.0, 3.0], dtype=np.float32)
    s_np = vals[rng.integers(0, len(vals), size=(w.batch * w.max_qo(), w.num_kv_heads,
                                                   w.max_pages()))]
    scores = torch.from_numpy(s_np).to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, _, _ = _select(run, scores, splits, write=False, dev_err=err)
    idx2, _ = run.topk(scores)
    out2 = run.attend(idx2, num_splits=splits)
    torch.cuda.synchronize()
    got = idx2.cpu().numpy()
    ind = c.qo_indptr.numpy()
    for r in range(w.batch):
        a, b = ind[r], ind[r + 1]
        e, _ = oracle.ladder_topk_request(s_np[a:b], int(c.lengths.kv[r]), w.top_k)
        assert np.array_equal(got[a:b], e.astype(np.int32)), f"request {r}"
    assert int(err.item()) == 0
    assert torch.equal(out[:run.n], out2[:run.n]), "fused and two-launch outputs differ"


def test_select_over_1024_pages_selects_in_its_own_launch():
    # 1100-page table: the selection runs as the standalone top-k into topk_idx, then the
    # sparse attention over it; without topk_idx the call is refused on the host
    w = W.LONG_FP8.scaled(name="pages_1100", batch=1, kv=("list", (140000,)), kv_capacity=140800,
                          top_k=8, num_q_heads=4, num_kv_heads=1)
    c = W.make_sparse_case(w)
    run = SparseRun(c)
    assert run.bt.shape[1] == 1100
    scores = run.scores()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, idx, cnt = _select(run, scores, 2, dev_err=err)
    torch.cuda.synchronize()
    ref = sparse_oracle(c)
    n = run.n
    assert np.array_equal(idx[:n].cpu().numpy(), ref["topk"][:n].astype(np.int32))
    assert np.array_equal(cnt[:n].cpu().numpy(), ref["count"][:n].astype(np.int32))
    ok, worst = tol_ok(out_numpy(out[:n]), ref["out"], "bf16")
    assert int(err.item()) == 0
    assert ok, worst
    with pytest.raises(sdv.SdvError):
        _select(run, scores, 1, write=False)


def test_select_top_k_beyond_valid_pages():
    # kv = 4, 128, 200 tokens: one or two valid pages, top_k = 8 -> -1 padding and
    # counts below top_k
    w = W.SPARSE_BF16.scaled(batch=3, qo=4, kv=("list", (4, 128, 200)), kv_capacity=512, top_k=8)
    c = W.make_sparse_case(w)
    run = SparseRun(c)
    out, idx, cnt = _select(run, run.scores(), 1)
    torch.cuda.synchronize()
    ref = sparse_oracle(c)
    n = run.n
    assert np.array_equal(idx[:n].cpu().numpy(), ref["topk"][:n].astype(np.int32))
    assert np.array_equal(cnt[:n].cpu().numpy(), ref["count"][:n].astype(np.int32))
    assert (idx[:n].cpu().numpy() == -1).any()
    ok, worst = tol_ok(out_numpy(out[:n]), ref["out"], "bf16")
    assert ok, worst


def test_select_flags_capacity_and_leaves_no_fault():
    c = W.make_sparse_case(SPARSE_S)
    run = SparseRun(c)
    scores = run.scores()
    kv_bad = c.kv_len.clone()
    kv_bad[1] = SPARSE_S.max_pages() * 128 + 1
    run.kv_len = kv_bad.to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    _select(run, scores, 2, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & sdv._lib.DEVERR_KV_CAPACITY


def test_select_host_errors():
    c = W.make_sparse_case(SPARSE_S)
    run = SparseRun(c)
    scores = run.scores()
    # the vector-ALU family needs an index buffer to hold the selection
    with pytest.raises(sdv.SdvError):
        _select(run, scores, 1, write=False, family=sdv.FAMILY_VALU)
    # more pages than any selection takes
    wide = torch.zeros(scores.shape[0], scores.shape[1], 4097, dtype=torch.float32, device=DEV)
    bt = torch.zeros(run.bt.shape[0], 4097, dtype=torch.int32, device=DEV)
    idx = torch.zeros(scores.shape[0], scores.shape[1], 4, dtype=torch.int32, device=DEV)
    with pytest.raises(sdv.SdvError):
        sdv.verify_attention_sparse_select(run.q, run.qo_indptr, run.kv_len, run.kv, bt, wide,
                                           max_qo_len=run.max_qo, top_k=4,
                                           softmax_scale=c.softmax_scale, topk_idx=idx)
