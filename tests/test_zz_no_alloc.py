"""GPU test of verify_attention_dense_view_noalloc, the entry point for callers that
cannot allocate: its split-KV partials live in the library's device scratch.  Two calls
in a row (the second smaller, so stale scratch contents from the first are present)
must equal verify_attention_dense_view with a caller workspace bit for bit, and the
small call must match the oracle."""
import numpy as np
import pytest
import torch

import speculative_decode_verify_p128_amd as sdv
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _parity import DEV, DenseRun, dense_oracle, out_numpy, tol_ok

SMALL = W.DENSE_BF16.scaled(name="noalloc_small", batch=5, kv=("uniform", 40, 1500),
                            kv_capacity=1536)
SMALL_FP8 = W.DENSE_BF16.scaled(name="noalloc_small_fp8", batch=3, kv=("uniform", 33, 900),
                                kv_capacity=1024, kv_dtype="fp8", num_q_heads=16)


def _view(run):
    w = run.c.w
    view, _ = sdv.kv_subpage_view_init(run.pool[w.root_page], run.bt, num_kv_heads=w.num_kv_heads,
                                       head_dim=w.head_dim, slot_stride=w.slot_stride,
                                       num_slots=run.c.num_slots, k_scale=run.c.k_scale,
                                       v_scale=run.c.v_scale, pool_index_scale=w.pool_index_scale,
                                       stage_offsets=False)
    return view


def _both(run, splits):
    view = _view(run)
    kw = dict(max_qo_len=run.max_qo, softmax_scale=run.c.softmax_scale, num_splits=splits)
    ref = sdv.verify_attention_dense_view(run.q, run.qo_indptr, run.kv_len, view, run.bt, **kw)
    got = torch.full_like(ref, float("nan"))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    sdv.verify_attention_dense_view_noalloc(run.q, run.qo_indptr, run.kv_len, view, run.bt,
                                            out=got, dev_err=err, **kw)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return got, ref


def test_noalloc_equals_workspace_entry_on_two_calls():
    print("\n[gpu] noalloc: full dense workload, 4 splits", flush=True)
    big = DenseRun(W.make_dense_case(W.DENSE_BF16, device=DEV))
    got, ref = _both(big, 4)
    assert torch.equal(got[:big.n], ref[:big.n])
    del big, got, ref
    print("[gpu] noalloc: smaller second call, 3 splits", flush=True)
    c = W.make_dense_case(SMALL)
    run = DenseRun(c)
    got, ref = _both(run, 3)
    assert torch.equal(got[:run.n], ref[:run.n])
    ok, worst = tol_ok(out_numpy(got[:run.n]), dense_oracle(c), "bf16")
    assert ok, worst


@pytest.mark.parametrize("splits", [1, 2, 16])
def test_noalloc_fp8_and_split_counts(splits):
    c = W.make_dense_case(SMALL_FP8)
    run = DenseRun(c)
    got, ref = _both(run, splits)
    assert torch.equal(got[:run.n], ref[:run.n])
    ok, worst = tol_ok(out_numpy(got[:run.n]), dense_oracle(c), "fp8")
    assert ok, worst


def test_noalloc_rejects_calls_beyond_the_scratch():
    c = W.make_dense_case(SMALL)
    run = DenseRun(c)
    view = _view(run)
    rows_cap = SMALL.batch * SMALL.max_qo()
    splits = 4096
    need = sdv.workspace_bytes(rows_cap, SMALL.num_q_heads, SMALL.head_dim, splits)
    assert need > sdv._lib.NOALLOC_SCRATCH_BYTES
    out = torch.empty((rows_cap, SMALL.num_q_heads, SMALL.head_dim), dtype=torch.bfloat16,
                      device=DEV)
    with pytest.raises(sdv.SdvError) as e:
        sdv.verify_attention_dense_view_noalloc(run.q, run.qo_indptr, run.kv_len, view, run.bt,
                                                max_qo_len=run.max_qo,
                                                softmax_scale=c.softmax_scale, num_splits=splits,
                                                out=out)
    assert e.value.status == sdv._lib.SDV_ERR_WORKSPACE
