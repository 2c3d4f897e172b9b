"""The one-launch entry points inside a captured HIP graph: the sparse step (proxy scores,
then verify_attention_sparse_select) and the dense draft step (verify_attention_dense_view)
are captured at short kv_len and replayed after the lengths change on the device (grown
to the tables' capacity, shrunk across page boundaries), with eager work between the
replays; every replay matches the oracle for the lengths it ran with."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_p128_amd as sdv
import workloads as W
from workloads import raw_numpy

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _parity import DEV, DenseRun, SparseRun, dense_oracle, out_numpy, tol_ok


def test_graph_replay_one_launch_paths():
    print("\n[gpu] graph replay of the one-launch paths", flush=True)
    w = W.SPARSE_BF16.scaled(batch=3, kv=("list", (700, 1500, 2600)), kv_capacity=2688, top_k=4)
    c = W.make_sparse_case(w)
    run = SparseRun(c)
    wd = W.DENSE_BF16.scaled(batch=3, kv=("list", (700, 1500, 2600)), kv_capacity=2688,
                             num_q_heads=16)
    d = W.make_dense_case(wd)
    drun = DenseRun(d)
    view, _ = sdv.kv_subpage_view_init(drun.pool[wd.root_page], drun.bt,
                                       num_kv_heads=wd.num_kv_heads, head_dim=wd.head_dim,
                                       slot_stride=wd.slot_stride, num_slots=d.num_slots,
                                       pool_index_scale=wd.pool_index_scale, stage_offsets=False)
    kv_dev = torch.tensor([300, 140, 2000], dtype=torch.int32, device=DEV)
    rows_cap = w.batch * w.max_qo()
    scores = torch.empty((rows_cap, w.num_kv_heads, w.max_pages()), dtype=torch.float32, device=DEV)
    idx = torch.empty((rows_cap, w.num_kv_heads, w.top_k), dtype=torch.int32, device=DEV)
    out = torch.empty((rows_cap, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    outd = torch.empty((rows_cap, wd.num_q_heads, wd.head_dim), dtype=torch.bfloat16, device=DEV)
    ws = sdv.alloc_workspace(rows_cap, w.num_q_heads, w.head_dim, 2, DEV)
    wsd = sdv.alloc_workspace(rows_cap, wd.num_q_heads, wd.head_dim, 4, DEV)

    def path():
        sdv.proxy_page_scores(run.q, run.qo_indptr, kv_dev, run.kv, run.bt, max_qo_len=4,
                              scores=scores)
        sdv.verify_attention_sparse_select(run.q, run.qo_indptr, kv_dev, run.kv, run.bt, scores,
                                           max_qo_len=4, top_k=w.top_k,
                                           softmax_scale=c.softmax_scale, num_splits=2,
                                           workspace=ws, out=out, topk_idx=idx)
        sdv.verify_attention_dense_view(drun.q, drun.qo_indptr, kv_dev, view, drun.bt,
                                        max_qo_len=4, softmax_scale=d.softmax_scale,
                                        num_splits=4, workspace=wsd, out=outd)

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
