"""GPU parity of verify_attention_dense_view: the draft view's P32 page indices computed
inside the attention launch from the block table.  Its output is compared with the
oracle (within tolerance) and bit for bit with the two-call path (kv_subpage_view_init,
then verify_attention_dense over the staged offsets) of the same kernel family, which
reads the same K/V blocks in the same order."""
import numpy as np
import pytest
import torch

import speculative_decode_verify_p128_amd as sdv
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _parity import DEV, DenseRun, dense_oracle, out_numpy, rows_of, tol_ok

TINY = W.TINY_FP32
DENSE_S = W.DENSE_BF16.scaled(name="dense_small", batch=3, kv=("uniform", 100, 900),
                              kv_capacity=1024)
DENSE_S_FP8 = W.DENSE_BF16.scaled(name="dense_small_fp8", batch=2, kv=("uniform", 33, 700),
                                  kv_capacity=768, kv_dtype="fp8", num_q_heads=16)
RAGGED_S = W.RAGGED_MIXED.scaled(name="ragged_small", batch=24,
                                 kv=("lognormal", 300, 1.0, 1, 2000, 0.25), kv_capacity=2048)
CASES = [TINY, DENSE_S, DENSE_S_FP8, RAGGED_S]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


def _view_only(run):
    w = run.c.w
    view, offs = sdv.kv_subpage_view_init(run.pool[w.root_page], run.bt,
                                          num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                          slot_stride=w.slot_stride, num_slots=run.c.num_slots,
                                          k_scale=run.c.k_scale, v_scale=run.c.v_scale,
                                          pool_index_scale=w.pool_index_scale,
                                          stage_offsets=False)
    assert offs is None
    return view


def _attend_view(run, view, num_splits, dev_err=None, family=0):
    return sdv.verify_attention_dense_view(run.q, run.qo_indptr, run.kv_len, view, run.bt,
                                           max_qo_len=run.max_qo,
                                           softmax_scale=run.c.softmax_scale,
                                           num_splits=num_splits, dev_err=dev_err, family=family)


@pytest.mark.parametrize("family", [0, 1, 3, 4, 5, 6])
@pytest.mark.parametrize("splits", [1, 2, 16])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_dense_view_parity(w, splits, family):
    c = W.make_dense_case(w)
    run = DenseRun(c)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = _attend_view(run, _view_only(run), splits, dev_err=err, family=family)
    view2, offs = run.view()
    out2 = run.attend(view2, offs, num_splits=splits, family=family)
    torch.cuda.synchronize()
    n = run.n
    ok, worst = tol_ok(out_numpy(out[:n]), dense_oracle(c), "f32" if w.kv_dtype == "f32" else "bf16")
    assert int(err.item()) == 0
    assert ok, f"max abs err {worst}"
    assert torch.equal(out[:n], out2[:n]), "fused and two-call outputs differ"


def test_dense_view_full_size_sampled():
    # the draft-layer benchmark workload in the benchmark's launch configuration: equal
    # to the two-call path bit for bit, and to the oracle on sampled requests
    w = W.DENSE_BF16
    c = W.make_dense_case(w, device=DEV)
    run = DenseRun(c)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = _attend_view(run, _view_only(run), w.num_splits, dev_err=err)
    view2, offs = run.view()
    out2 = run.attend(view2, offs, num_splits=w.num_splits)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(out[:run.n], out2[:run.n])
    got = out_numpy(out[:run.n])
    del run, view2, offs, out, out2
    for f in ("q", "qo_indptr", "kv_len", "block_table", "pool"):
        setattr(c, f, getattr(c, f).cpu())
    req = [int(np.argmax(c.lengths.kv)), int(np.argmin(c.lengths.kv)), 5]
    ref = dense_oracle(c, requests=req)
    rows = rows_of(c, req)
    ok, worst = tol_ok(got[rows], ref[rows], "bf16")
    assert ok, worst


def test_dense_view_flags_slots_outside_the_view():
    c = W.make_dense_case(DENSE_S)
    run = DenseRun(c)
    bt = run.bt.clone()
    bt[1, 0] = c.num_slots          # one past the last slot
    run.bt = bt
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    _attend_view(run, _view_only(run), 2, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & sdv._lib.DEVERR_PAGE_RANGE
