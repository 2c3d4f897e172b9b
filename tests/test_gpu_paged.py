"""GPU parity of dense verify attention over ordinary head-major P128 pages (the target's
dense layers with the ladder mask) against the oracle: small cases element by element
over splits and the matrix-core kernel families, poison in positions no row may see,
page-index flags, and the full benchmark size on sampled requests."""
import numpy as np
import pytest
import torch

import speculative_decode_verify_p128_amd as sdv
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _parity import DEV, PagedRun, out_numpy, paged_oracle, rows_of, tol_ok

PAGED_S = W.PAGED_BF16.scaled(name="paged_small", batch=3, kv=("uniform", 500, 3000),
                              kv_capacity=3072)
PAGED_FP8 = W.LONG_FP8.scaled(name="paged_fp8", batch=2, kv=("fixed", 5000), kv_capacity=5120)
PAGED_RAGGED = W.RAGGED_MIXED.scaled(name="paged_ragged", batch=24,
                                     kv=("lognormal", 300, 1.0, 1, 2000, 0.25), kv_capacity=2048)
PAGED_D64 = W.PAGED_BF16.scaled(name="paged_d64", batch=3, kv=("uniform", 130, 1000),
                                kv_capacity=1024, head_dim=64, num_q_heads=8, num_kv_heads=2)
PAGED_G16 = W.PAGED_BF16.scaled(name="paged_g16", batch=2, kv=("uniform", 40, 900),
                                kv_capacity=1024, num_q_heads=64)
CASES = [PAGED_S, PAGED_FP8, PAGED_RAGGED, PAGED_D64, PAGED_G16]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


@pytest.mark.parametrize("family", [0, 3, 4, 5, 6])
@pytest.mark.parametrize("splits", [1, 2, 16])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_paged_parity(w, splits, family):
    c = W.make_sparse_case(w)
    run = PagedRun(c)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run.attend_paged(num_splits=splits, dev_err=err, family=family)
    torch.cuda.synchronize()
    ref = paged_oracle(c)
    ok, worst = tol_ok(out_numpy(out[:run.n]), ref, "bf16")
    assert int(err.item()) == 0
    assert ok, f"max abs err {worst}"


@pytest.mark.parametrize("family", [0, 3, 4, 5, 6])
def test_paged_poison_never_read(family):
    """NaN beyond every request's kv_len in its last page and in every page it does not
    own: no output may see them."""
    c = W.make_sparse_case(PAGED_S, poison=True)
    for pool in (c.k_pool, c.v_pool):
        for r, kv in enumerate(c.lengths.kv):
            kv = int(kv)
            if kv % 128:
                pool[int(c.block_table[r, kv // 128]), :, kv % 128:, :] = float("nan")
    run = PagedRun(c)
    out = run.attend_paged(num_splits=2, family=family)
    torch.cuda.synchronize()
    ok, worst = tol_ok(out_numpy(out[:run.n]), paged_oracle(c), "bf16")
    assert ok, worst


@pytest.mark.parametrize("qo,kvs", [(1, [1, 2, 128, 129]), (4, [4, 5, 128, 129])])
def test_paged_decode_and_minimum_lengths(qo, kvs):
    """qo_len = 1 is ordinary decode attention; kv_len = qo_len attends only the verify
    tokens; exact page multiples and one past them."""
    w = PAGED_S.scaled(name=f"paged_edges_{qo}", batch=4, qo=qo, kv=("fixed", 256))
    c = W.make_sparse_case(w)
    c.lengths.kv[:] = np.array(kvs)
    c.kv_len[:] = torch.tensor(kvs, dtype=torch.int32)
    run = PagedRun(c)
    out = run.attend_paged(num_splits=2)
    torch.cuda.synchronize()
    ok, worst = tol_ok(out_numpy(out[:run.n]), paged_oracle(c), "bf16")
    assert ok, worst


def test_paged_bad_page_is_flagged():
    c = W.make_sparse_case(PAGED_S)
    run = PagedRun(c)
    bt = c.block_table.clone()
    bt[1, 0] = c.k_pool.shape[0] + 7
    run.bt = bt.to(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    run.attend_paged(dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & sdv._lib.DEVERR_PAGE_RANGE


def test_paged_full_size_sampled():
    w = W.PAGED_BF16
    print(f"\n[gpu] paged full {w.name}", flush=True)
    c = W.make_sparse_case(w, device=DEV)
    run = PagedRun(c)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run.attend_paged(num_splits=w.num_splits, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = out_numpy(out[:run.n])
    del run, out
    for f in ("q", "qo_indptr", "kv_len", "block_table", "k_pool", "v_pool"):
        setattr(c, f, getattr(c, f).cpu())
    kv = c.lengths.kv
    req = sorted({int(np.argmin(kv)), int(np.argmax(kv)), 0, len(kv) // 2, len(kv) - 1})
    ref = paged_oracle(c, requests=req)
    rows = rows_of(c, req)
    ok, worst = tol_ok(got[rows], ref[rows], "bf16")
    assert ok, worst
