"""GPU parity of the persistent dense kernels, which give every workgroup an equal range
of 32-token blocks over all (request, KV head) pairs laid end to end, so that a split
slot is a consecutive piece of a pair: many short requests (one workgroup covers many
pairs), few long ones (a pair spans up to num_splits workgroups), requests with
inconsistent lengths among valid ones, and both dense sources (the P32 view of the
draft layer and head-major P128 pages)."""
import functools

import numpy as np
import pytest
import torch

import speculative_decode_verify_p128_amd as sdv
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _parity import (DEV, DenseRun, PagedRun, dense_oracle, out_numpy, paged_oracle,
                         rows_of, tol_ok)

FAMILIES = [5, 6]   # the per-wave and the LDS-ring kernels under the persistent partition

MANY_SHORT_VIEW = W.DENSE_BF16.scaled(name="many_short_view", batch=600, kv=("uniform", 4, 100),
                                      kv_capacity=128, num_q_heads=16)
# 64 and 32 query rows per pair: the row tiles whose ranges hold fewer finished pieces in
# registers than these ranges have pieces, so later pieces are written at once
MANY_SHORT_VIEW64 = W.DENSE_BF16.scaled(name="many_short_view64", batch=600, kv=("uniform", 4, 100),
                                        kv_capacity=128)
MANY_SHORT_VIEW32 = W.DENSE_BF16.scaled(name="many_short_view32", batch=600, kv=("uniform", 4, 100),
                                        kv_capacity=128, num_q_heads=32)
FEW_LONG_VIEW = W.DENSE_BF16.scaled(name="few_long_view", batch=2, kv=("uniform", 3000, 6000),
                                    kv_capacity=6144)
MANY_SHORT_PAGED = W.PAGED_BF16.scaled(name="many_short_paged", batch=600, kv=("uniform", 4, 100),
                                       kv_capacity=128)
FEW_LONG_PAGED = W.PAGED_BF16.scaled(name="few_long_paged", batch=2, kv=("uniform", 3000, 6000),
                                     kv_capacity=6144, num_q_heads=64)
RAGGED_PAGED_FP8 = W.RAGGED_MIXED.scaled(name="ragged_paged_fp8", batch=40, kv_dtype="fp8",
                                         kv=("lognormal", 400, 1.0, 1, 3000, 0.25),
                                         kv_capacity=3072)


@functools.lru_cache(maxsize=None)
def _dense(w):
    c = W.make_dense_case(w)
    return c, dense_oracle(c)


@functools.lru_cache(maxsize=None)
def _paged(w):
    c = W.make_sparse_case(w)
    return c, paged_oracle(c)


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("splits", [2, 3, 16])
@pytest.mark.parametrize("w", [MANY_SHORT_VIEW, MANY_SHORT_VIEW64, MANY_SHORT_VIEW32, FEW_LONG_VIEW],
                         ids=lambda w: w.name)
def test_persist_view_parity(w, splits, family):
    c, ref = _dense(w)
    run = DenseRun(c)
    view, offs = run.view()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run.attend(view, offs, num_splits=splits, dev_err=err, family=family)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ok, worst = tol_ok(out_numpy(out[:run.n]), ref, "bf16")
    assert ok, f"max abs err {worst}"


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("splits", [2, 3, 16])
@pytest.mark.parametrize("w", [MANY_SHORT_PAGED, FEW_LONG_PAGED, RAGGED_PAGED_FP8],
                         ids=lambda w: w.name)
def test_persist_paged_parity(w, splits, family):
    c, ref = _paged(w)
    run = PagedRun(c)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run.attend_paged(num_splits=splits, dev_err=err, family=family)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ok, worst = tol_ok(out_numpy(out[:run.n]), ref, "bf16")
    assert ok, f"max abs err {worst}"


# one long request beside many short ones at two splits: the range length follows the
# long request, so a range holds more pieces than one plan takes and is planned again
_MIXED_KV = (6000,) + tuple(4 + (7 * i) % 33 for i in range(1, 300))
MIXED_VIEW64 = W.DENSE_BF16.scaled(name="mixed_view64", batch=300, kv=("list", _MIXED_KV),
                                   kv_capacity=6016)
MIXED_VIEW16 = W.DENSE_BF16.scaled(name="mixed_view16", batch=300, kv=("list", _MIXED_KV),
                                   kv_capacity=6016, num_q_heads=16)


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("w", [MIXED_VIEW64, MIXED_VIEW16], ids=lambda w: w.name)
def test_persist_view_replanned_ranges(w, family):
    c, ref = _dense(w)
    run = DenseRun(c)
    view, offs = run.view()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run.attend(view, offs, num_splits=2, dev_err=err, family=family)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ok, worst = tol_ok(out_numpy(out[:run.n]), ref, "bf16")
    assert ok, f"max abs err {worst}"


@pytest.mark.parametrize("family", FAMILIES)
def test_persist_inconsistent_requests_flagged_others_exact(family):
    """Request 2 shorter than its verify tokens, request 5 beyond the table's capacity:
    both are flagged and count as empty; every other request matches the oracle."""
    w = W.PAGED_BF16.scaled(name="persist_flags", batch=8, kv=("uniform", 200, 2000),
                            kv_capacity=2048)
    c = W.make_sparse_case(w)
    run = PagedRun(c)
    kv_bad = c.kv_len.clone()
    kv_bad[2] = 2
    kv_bad[5] = w.max_pages() * 128 + 1
    run.kv_len = kv_bad.to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run.attend_paged(num_splits=4, dev_err=err, family=family)
    torch.cuda.synchronize()
    e = int(err.item())
    assert e & sdv._lib.DEVERR_QO_LEN and e & sdv._lib.DEVERR_KV_CAPACITY
    good = [r for r in range(w.batch) if r not in (2, 5)]
    rows = rows_of(c, good)
    ok, worst = tol_ok(out_numpy(out[:run.n])[rows], paged_oracle(c, requests=good)[rows], "bf16")
    assert ok, worst


@pytest.mark.parametrize("family", FAMILIES)
def test_persist_matches_per_split_kernel_at_benchmark_size(family):
    """The dense benchmark configuration: the persistent kernel and the per-split kernel
    agree to the bf16 tolerance on every row, and sampled requests match the oracle."""
    w = W.DENSE_BF16
    c = W.make_dense_case(w, device=DEV)
    run = DenseRun(c)
    view, offs = run.view()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = run.attend(view, offs, num_splits=8, dev_err=err, family=family)
    ref_gpu = run.attend(view, offs, num_splits=8, family=sdv.FAMILY_WAVES)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ok, worst = tol_ok(out_numpy(got[:run.n]), out_numpy(ref_gpu[:run.n]), "bf16")
    assert ok, worst
    got = out_numpy(got[:run.n])
    del run, ref_gpu
    for f in ("q", "qo_indptr", "kv_len", "block_table", "pool"):
        setattr(c, f, getattr(c, f).cpu())
    kv = c.lengths.kv
    req = sorted({int(np.argmin(kv)), int(np.argmax(kv)), 0, len(kv) - 1})
    rows = rows_of(c, req)
    ok, worst = tol_ok(got[rows], dense_oracle(c, requests=req)[rows], "bf16")
    assert ok, worst
