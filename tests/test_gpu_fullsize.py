"""GPU parity at the full benchmark sizes and launch configurations (the splits the
benchmark uses), checked on sampled requests that the oracle computes one by one.
Inputs are generated on the GPU with a seeded generator and copied to the host for
the oracle (same bytes on both sides)."""
import numpy as np
import pytest
import torch

import speculative_decode_verify_p128_amd as sdv
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _parity import (DEV, DenseRun, SparseRun, dense_oracle, out_numpy, rows_of,
                         sparse_oracle, tol_ok)


def _sample(kv, k, seed):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(len(kv), size=min(k, len(kv)), replace=False).tolist())
    pick |= {int(np.argmax(kv)), int(np.argmin(kv))}
    return sorted(pick)


def _to_cpu(case):
    for f in ("q", "qo_indptr", "kv_len", "block_table", "pool", "k_pool", "v_pool"):
        if hasattr(case, f):
            setattr(case, f, getattr(case, f).cpu())
    return case


@pytest.mark.parametrize("w", [W.DENSE_BF16, W.RAGGED_MIXED], ids=lambda w: w.name)
def test_dense_full_size_sampled(w):
    print(f"\n[gpu] dense full {w.name}", flush=True)
    c = W.make_dense_case(w, device=DEV)
    run = DenseRun(c)
    view, offs = run.view()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = run.attend(view, offs, num_splits=w.num_splits, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = out_numpy(out[:run.n])
    del run, view, offs, out
    c = _to_cpu(c)
    req = _sample(c.lengths.kv, 3, 5)
    ref = dense_oracle(c, requests=req)
    rows = rows_of(c, req)
    ok, worst = tol_ok(got[rows], ref[rows], "bf16")
    assert ok, worst


@pytest.mark.parametrize("w", [W.SPARSE_BF16, W.LONG_FP8, W.RAGGED_MIXED], ids=lambda w: w.name)
def test_sparse_full_size_sampled(w):
    print(f"\n[gpu] sparse full {w.name}", flush=True)
    c = W.make_sparse_case(w, device=DEV)
    run = SparseRun(c)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    scores = run.scores(dev_err=err)
    idx, cnt = run.topk(scores, dev_err=err)
    out = run.attend(idx, num_splits=w.num_splits, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    s_np, i_np, o_np = scores.cpu().numpy(), idx.cpu().numpy(), out_numpy(out[:run.n])
    del run, scores, idx, out
    c = _to_cpu(c)
    req = _sample(c.lengths.kv, 2, 6)
    ref = sparse_oracle(c, requests=req)
    ind = c.qo_indptr.numpy()
    for r in req:
        a, b = ind[r], ind[r + 1]
        npg = -(-int(c.lengths.kv[r]) // 128)
        assert np.array_equal(s_np[a:b, :, :npg].view(np.uint32),
                              ref["scores"][a:b, :, :npg].view(np.uint32)), f"scores r={r}"
        assert np.array_equal(i_np[a:b], ref["topk"][a:b].astype(np.int32)), f"topk r={r}"
    rows = rows_of(c, req)
    ok, worst = tol_ok(o_np[rows], ref["out"][rows], "bf16")
    assert ok, worst


@pytest.mark.parametrize("w", [W.SPARSE_BF16, W.LONG_FP8, W.RAGGED_MIXED], ids=lambda w: w.name)
def test_select_full_size_sampled(w):
    """The benchmark's sparse step (proxy scores, then selection + attention in one
    launch) at full size and the workload's split count: its selection (written out) is
    the oracle's on sampled requests and its output within tolerance."""
    print(f"\n[gpu] fused select full {w.name}", flush=True)
    c = W.make_sparse_case(w, device=DEV)
    run = SparseRun(c)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    scores = run.scores(dev_err=err)
    rows_cap = w.batch * w.max_qo()
    idx = torch.full((rows_cap, w.num_kv_heads, w.top_k), -7, dtype=torch.int32, device=DEV)
    out = sdv.verify_attention_sparse_select(run.q, run.qo_indptr, run.kv_len, run.kv, run.bt,
                                             scores, max_qo_len=run.max_qo, top_k=w.top_k,
                                             softmax_scale=c.softmax_scale,
                                             num_splits=w.num_splits, topk_idx=idx, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    i_np, o_np = idx.cpu().numpy(), out_numpy(out[:run.n])
    del run, scores, idx, out
    c = _to_cpu(c)
    req = _sample(c.lengths.kv, 2, 7)
    ref = sparse_oracle(c, requests=req)
    ind = c.qo_indptr.numpy()
    for r in req:
        a, b = ind[r], ind[r + 1]
        assert np.array_equal(i_np[a:b], ref["topk"][a:b].astype(np.int32)), f"topk r={r}"
    rows = rows_of(c, req)
    ok, worst = tol_ok(o_np[rows], ref["out"][rows], "bf16")
    assert ok, worst
