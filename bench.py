"""Benchmark of the verify path on one MI355X.

A step is one pass of the block-sparse target-layer verify path over one batch:
proxy page scores, then the ladder top-k and the sparse verify attention in one launch
(+ split-KV combine), on the sparse bf16 workload (batch 64, qo_len 4, 16/4 heads,
head_dim 128, kv_len uniform in [4096, 32768], top-k 16).  The same path as three
launches (standalone top-k) is timed after it and reported under "unfused".  Inputs are
generated on the GPU from a seed and are resident in HBM before timing starts.  The
dense draft-layer path (dense verify attention through the P32 view, its page indices
computed in the same launch; batch 32, qo_len 4, 64/4 heads, kv_len uniform in
[1024, 8192]) is timed in the same run and reported under "dense".

Prints one JSON line.  The step time comes from one pair of HIP events around each
timed step; per-kernel durations come from HIP events recorded on the launch stream
around every kernel in a second timed loop of the same steps (an event between two
launches delays the second, so it stays out of the step time).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify tokens/sec + achieved HBM GB/s (% of peak), sparse paged GQA qo_len=4"
HBM_PEAK_GBS = 8000.0
ACCEPT_VOCAB = 131072          # synthetic vocabulary size of the acceptance line


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--splits", type=int, default=None, help="override sparse num_splits")
    p.add_argument("--dense-splits", type=int, default=None)
    p.add_argument("--family", type=int, default=0,
                   help="attention kernels (through the cross-check library when nonzero): "
                        "0 default, 1 vector-ALU, 3 per-wave LDS stream, 4 workgroup LDS ring, "
                        "5 persistent per-wave, 6 persistent ring")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-paged", action="store_true")
    p.add_argument("--paged-splits", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=64, help="requests in the oracle sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a 1 GiB device copy (for memory-counter calibration)")
    p.add_argument("--no-probe", action="store_true", help="skip the streaming-read probe")
    p.add_argument("--graph", action="store_true",
                   help="time the headline step as one HIP graph replay instead of eager launches")
    p.add_argument("--warm", action="store_true",
                   help="no cache-evicting fill between steps (warm-cache numbers)")
    p.add_argument("--dense-two-call", action="store_true",
                   help="also time the draft-layer step as two calls (view offsets, then "
                        "attention over them), reported under dense.two_call")
    p.add_argument("--long-splits", type=int, default=None)
    p.add_argument("--ragged-splits", type=int, default=None, help="ragged sparse num_splits")
    p.add_argument("--ragged-dense-splits", type=int, default=None)
    p.add_argument("--no-extra-configs", action="store_true",
                   help="skip the long-context fp8 and ragged-batch lines")
    p.add_argument("--only", default=None,
                   help="comma list of sections to run (sparse, dense, paged, long_fp8, ragged, "
                        "staging, transfer, accept); the headline sparse line always runs")
    p.add_argument("--no-unfused", action="store_true",
                   help="skip timing the three-launch step (proxy, standalone top-k, sparse "
                        "attention over its indices) reported under 'unfused'")
    return p.parse_args()


def sparse_algorithmic_bytes(case, idx_np):
    """Bytes each sparse-path kernel must move (no re-reads, no partials)."""
    w = case.w
    e = {"f32": 4, "bf16": 2, "fp8": 1}[w.kv_dtype]
    eq = {"f32": 4, "bf16": 2}[w.q_dtype]
    d, Hq, Hkv = w.head_dim, w.num_q_heads, w.num_kv_heads
    qo, kv = case.lengths.qo, case.lengths.kv
    ind = case.lengths.qo_indptr
    rows = int(qo.sum())
    q_bytes = rows * Hq * d * eq
    n_pages = -(-kv // 128)
    # proxy: every valid K row once, Q, the block table, the written scores
    proxy = int(kv.sum()) * Hkv * d * e + q_bytes + int(n_pages.sum()) * 4 + \
        int((qo * n_pages).sum()) * Hkv * 4
    # top-k: valid score entries read, indices written
    nv_sum = 0
    for r in range(len(kv)):
        b = kv[r] - qo[r] + np.arange(qo[r]) + 1
        nv_sum += int((-(-b // 128)).sum())
    topk = nv_sum * Hkv * 4 + rows * Hkv * w.top_k * 4
    scores_read = nv_sum * Hkv * 4
    index_bytes = rows * Hkv * w.top_k * 4
    # sparse: valid K and V rows of the distinct pages any token of (r, h) selected
    kv_rows = 0
    for r in range(len(kv)):
        sel = idx_np[ind[r]:ind[r + 1]]                      # [qo, Hkv, K]
        for h in range(Hkv):
            pages = np.unique(sel[:, h, :])
            pages = pages[pages >= 0]
            kv_rows += int(np.minimum(128, kv[r] - 128 * pages).sum())
    sparse = kv_rows * d * e * 2 + q_bytes + rows * Hq * d * eq + rows * Hkv * w.top_k * 4 + \
        int(n_pages.sum()) * 4
    rowexp = 0
    for r in range(len(kv)):
        sel = idx_np[ind[r]:ind[r + 1]]
        for t in range(qo[r]):
            for h in range(Hkv):
                pages = sel[t, h][sel[t, h] >= 0]
                rowexp += int(np.minimum(128, kv[r] - 128 * pages).sum())
    # in-kernel selection: the valid scores read in place of the indices
    select = sparse - index_bytes + scores_read
    return {"proxy": proxy, "topk": topk, "sparse": sparse, "select": select,
            "sparse_row_expanded_kv": rowexp * d * e * 2}


def dense_algorithmic_bytes(case, staged_offsets=False):
    """Every valid K and V row once, Q and O, and the page indices: the block-table
    entries (one per 128-token page) when the attention computes the view's indices,
    the staged K and V offsets (one each per 32-token sub-page) otherwise."""
    w = case.w
    e = {"f32": 4, "bf16": 2, "fp8": 1}[w.kv_dtype]
    eq = {"f32": 4, "bf16": 2}[w.q_dtype]
    rows = case.lengths.total_q
    kv = case.lengths.kv
    idx = int((-(-kv // 32)).sum()) * 2 * 4 if staged_offsets else int((-(-kv // 128)).sum()) * 4
    return int(kv.sum()) * w.num_kv_heads * w.head_dim * e * 2 + \
        2 * rows * w.num_q_heads * w.head_dim * eq + idx


# Sources that decide each timed kernel's memory traffic: a counter summary taken on
# other sources no longer describes the kernel.
KERNEL_SOURCES = {
    "proxy_page_scores": ("k_proxy.hip", "device.h"),
    "ladder_topk_pages": ("k_topk.hip", "device.h", "internal.h"),
    "verify_attention_sparse": ("k_attn_waves.hip", "mfma_attn.h", "sparse_union.h", "k_small.hip",
                                "device.h", "internal.h", "sdv_api.cpp"),
    "verify_attention_sparse_select": ("k_attn_waves.hip", "mfma_attn.h", "sparse_union.h",
                                       "k_small.hip", "device.h", "internal.h", "sdv_api.cpp"),
    "verify_attention_dense": ("k_attn_stream.hip", "k_attn_flat.hip", "mfma_attn.h",
                               "k_small.hip", "device.h", "internal.h", "sdv_api.cpp"),
    "verify_attention_dense_view": ("k_attn_stream.hip", "k_attn_flat.hip", "mfma_attn.h",
                                    "k_small.hip", "device.h", "internal.h", "sdv_api.cpp"),
    "verify_attention_paged": ("k_attn_waves.hip", "mfma_attn.h", "k_small.hip", "device.h",
                               "internal.h", "sdv_api.cpp"),
    "greedy_accept": ("k_accept.hip", "device.h", "internal.h", "sdv_api.cpp"),
    "copy_descriptors": ("k_copy.hip", "device.h", "internal.h", "sdv_api.cpp"),
}


def paged_algorithmic_bytes(case):
    """Dense over head-major pages: every valid K and V row of every (request, KV head)
    once, Q read, O written, one block-table entry per page."""
    w = case.w
    e = {"f32": 4, "bf16": 2, "fp8": 1}[w.kv_dtype]
    eq = {"f32": 4, "bf16": 2}[w.q_dtype]
    kv = case.lengths.kv
    rows = case.lengths.total_q
    return int(kv.sum()) * w.num_kv_heads * w.head_dim * e * 2 + \
        2 * rows * w.num_q_heads * w.head_dim * eq + int((-(-kv // 128)).sum()) * 4


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "speculative_decode_verify_p128_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, src_hash):
    """HBM bytes per launch from a committed counter summary, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def time_steps(step_fns, steps, warmup, torch, flush=None, stats=None):
    """Runs warmup + timed steps.  With `flush`, a cache-evicting fill runs before every
    step outside the timed span.  The step time comes from one pair of events around each
    step's launches; an event recorded between two launches delays the second by several
    microseconds, so when a step has more than one launch the per-launch durations come
    from a second timed pass with events around every launch (`stats`, if given, receives
    that pass's mean step time).  Returns (ms per step, per-launch stats, wall seconds
    of the first pass)."""
    n = len(step_fns)

    def run_pass(per_launch):
        for _ in range(warmup):
            if flush:
                flush()
            for _, fn in step_fns:
                fn()
        torch.cuda.synchronize()
        marks = n + 1 if per_launch else 2
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(marks)] for _ in range(steps)]
        t0 = time.perf_counter()
        for s in range(steps):
            if flush:
                flush()
            ev[s][0].record()
            for i, (_, fn) in enumerate(step_fns):
                fn()
                if per_launch:
                    ev[s][i + 1].record()
            if not per_launch:
                ev[s][1].record()
        torch.cuda.synchronize()
        return ev, time.perf_counter() - t0

    ev, wall = run_pass(per_launch=(n == 1))
    step_ms = [ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)]
    if n > 1:
        ev, _ = run_pass(per_launch=True)
        if stats is not None:
            stats["ms_per_step_with_launch_events"] = float(np.mean(
                [ev[s][0].elapsed_time(ev[s][n]) for s in range(steps)]))
    per = {}
    for i, (name, _) in enumerate(step_fns):
        ts = [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]
        per[name] = {"avg_us": 1e3 * float(np.mean(ts)), "min_us": 1e3 * float(np.min(ts)),
                     "p10_us": 1e3 * float(np.percentile(ts, 10)),
                     "p50_us": 1e3 * float(np.median(ts)),
                     "p90_us": 1e3 * float(np.percentile(ts, 90))}
    return float(np.mean(step_ms)), per, wall


def time_graph(step_fns, steps, warmup, torch, flush=None):
    """The same step captured once as a HIP graph and replayed: the step time is the
    event span around each replay, the cache-evicting fill (if any) runs eagerly before
    it, outside the span.  Returns the mean step time in ms."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _, fn in step_fns:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _, fn in step_fns:
            fn()
    for _ in range(warmup):
        if flush:
            flush()
        graph.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        if flush:
            flush()
        e0.record()
        graph.replay()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    del graph
    return ms


def host_cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, n_req):
    """The oracle, untuned, on a bounded sample of the same workload, one thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    from workloads import raw_numpy
    w = case.w
    req = list(range(min(n_req, w.batch)))
    q_raw = raw_numpy(case.q)
    kp, vp = raw_numpy(case.k_pool), raw_numpy(case.v_pool)
    bt = case.block_table.cpu().numpy()
    ind = case.qo_indptr.cpu().numpy()
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.sparse_verify_case(q_raw, w.q_dtype, ind, case.lengths.kv, kp, vp, w.kv_dtype, bt,
                                  case.k_scale, case.v_scale, w.top_k, case.softmax_scale,
                                  w.max_pages(), requests=req)
        dt = time.perf_counter() - t0
    toks = int(sum(case.lengths.qo[r] for r in req))
    kvs = [int(case.lengths.kv[r]) for r in req]
    return {"value": toks / dt, "unit": "verify tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(req)} of {w.batch} requests ({toks} verify tokens, {sum(kvs)} kv "
                      f"tokens, kv_len {min(kvs)}..{max(kvs)}) through proxy scores, top-k and "
                      f"sparse attention, one thread; {dt:.1f} s"}


def _oracle_worker_init():
    """Worker start-up (untimed): one BLAS/OpenMP thread, the oracle imported."""
    from threadpoolctl import threadpool_limits
    import oracle  # noqa: F401
    threadpool_limits(limits=1)


def _oracle_worker(task):
    """One process of the all-cores oracle timing: attaches the shared inputs and runs the
    oracle, one thread, on its share of the requests."""
    from multiprocessing import shared_memory
    from threadpoolctl import threadpool_limits
    import oracle
    names, shapes, dtypes, meta, req = task
    shms = [shared_memory.SharedMemory(name=n) for n in names]
    try:
        q_raw, kp, vp, bt, ind, kvl = [np.ndarray(sh, dtype=dt, buffer=m.buf)
                                       for m, sh, dt in zip(shms, shapes, dtypes)]
        if req:
            with threadpool_limits(limits=1):
                oracle.sparse_verify_case(q_raw, meta["q_dtype"], ind, kvl, kp, vp, meta["kv_dtype"],
                                          bt, meta["k_scale"], meta["v_scale"], meta["top_k"],
                                          meta["softmax_scale"], meta["max_pages"], requests=req)
        del q_raw, kp, vp, bt, ind, kvl
    finally:
        for m in shms:
            m.close()
    return len(req)


def start_oracle_pool(max_procs=16):
    """The worker processes of the all-cores oracle timing, started before this process
    touches the GPU (new processes are never started from a GPU-initialised one), with
    one BLAS/OpenMP thread each."""
    import multiprocessing as mp
    procs = max(1, min(max_procs, len(os.sched_getaffinity(0))))
    threads_env = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in threads_env}
    os.environ.update({k: "1" for k in threads_env})   # inherited by the spawned workers
    try:
        pool = mp.get_context("spawn").Pool(procs, initializer=_oracle_worker_init)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return pool, procs


def cpu_baseline_all_cores(case, n_req, pool, procs):
    """The same oracle sample split over the pool's processes, one per core (requests
    dealt round-robin after sorting by length); inputs shared; the second of two identical
    passes is timed (the first one pays the workers' first-use costs)."""
    from multiprocessing import shared_memory
    from workloads import raw_numpy
    w = case.w
    req = sorted(range(min(n_req, w.batch)), key=lambda r: -int(case.lengths.kv[r]))
    procs = max(1, min(procs, len(req)))
    arrays = [raw_numpy(case.q), raw_numpy(case.k_pool), raw_numpy(case.v_pool),
              case.block_table.cpu().numpy(), case.qo_indptr.cpu().numpy(),
              np.asarray(case.lengths.kv)]
    shms = []
    try:
        for a in arrays:
            m = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
            np.ndarray(a.shape, dtype=a.dtype, buffer=m.buf)[...] = a
            shms.append(m)
        meta = {"q_dtype": w.q_dtype, "kv_dtype": w.kv_dtype, "k_scale": case.k_scale,
                "v_scale": case.v_scale, "top_k": w.top_k, "softmax_scale": case.softmax_scale,
                "max_pages": w.max_pages()}
        base = ([m.name for m in shms], [a.shape for a in arrays], [a.dtype for a in arrays], meta)
        tasks = [base + (req[i::procs],) for i in range(procs)]
        pool.map(_oracle_worker, tasks, chunksize=1)   # untimed: workers' first pass
        t0 = time.perf_counter()
        pool.map(_oracle_worker, tasks, chunksize=1)
        dt = time.perf_counter() - t0
    finally:
        for m in shms:
            m.close()
            m.unlink()
    toks = int(sum(case.lengths.qo[r] for r in req))
    return {"value": toks / dt, "unit": "verify tokens/s", "cores": procs, "kind": "oracle",
            "sample": f"the same {len(req)} requests over {procs} processes, one thread each; "
                      f"{dt:.2f} s"}


def attainable_read_gbs(torch, sdv, dev, gib=4):
    """Best rate of the streaming-read probe over a buffer far larger than the caches."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    best = 0.0
    for blocks in (1024, 2048, 4096, 8192):
        sink = torch.zeros(blocks, dtype=torch.int32, device=dev)
        sdv.read_probe(buf, sink, blocks)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(5):
            sdv.read_probe(buf, sink, blocks)
        e.record()
        torch.cuda.synchronize()
        best = max(best, 5 * buf.numel() / (s.elapsed_time(e) * 1e-3) / 1e9)
    del buf
    return best


def units_read_gbs(torch, sdv, dev, lists, flush, reps=5):
    """Best cold rate of the unit-list probe over a kernel's own gather list, given as
    (base tensor, int64 unit indices, unit bytes) per buffer, read back to back."""
    best = 0.0
    nbytes = sum(u.numel() * ub for _, u, ub in lists)
    for blocks in (1024, 2048, 4096):
        sink = torch.zeros(blocks, dtype=torch.int32, device=dev)
        tot = 0.0
        for it in range(reps + 1):
            if flush:
                flush()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for base, units, unit_bytes in lists:
                sdv.read_units_probe(base, units, unit_bytes, sink, blocks)
            e.record()
            torch.cuda.synchronize()
            if it:
                tot += s.elapsed_time(e)
        best = max(best, nbytes / (tot / reps * 1e-3) / 1e9)
    return best


def sparse_gather_units(case, idx_np, torch, dev):
    """The proxy's gather list (K of every valid page of every (request, KV head)) and the
    sparse attention's (K and V of the pages any token of the pair chose), as 16 KiB
    units of the head-major P128 pools (a page's head is two units)."""
    w = case.w
    Hkv = w.num_kv_heads
    bt = case.block_table.cpu().numpy()
    ind = case.qo_indptr.cpu().numpy()
    assert w.head_dim * 2 * 128 == 2 * 16384 and case.k_pool.is_contiguous()
    proxy, sel = [], []
    for r in range(w.batch):
        n = (int(case.lengths.kv[r]) + 127) // 128
        phys = bt[r, :n].astype(np.int64)
        for h in range(Hkv):
            for half in (0, 1):
                proxy.append((phys * Hkv + h) * 2 + half)
            chosen = np.unique(idx_np[ind[r]:ind[r + 1], h, :])
            chosen = chosen[chosen >= 0]
            for half in (0, 1):
                sel.append((bt[r, chosen].astype(np.int64) * Hkv + h) * 2 + half)
    t = lambda a: torch.from_numpy(np.concatenate(a)).to(dev)  # noqa: E731
    return t(proxy), t(sel)


def sparse_config_line(torch, sdv, W, w, dev, args, flush, fam, splits=None):
    """The sparse target-layer step on workload w: proxy scores, then the ladder top-k
    and sparse attention (+ the split-KV combine) either in one launch (selection inside
    the attention workgroups) or as a standalone top-k launch and the attention over its
    indices; both are timed and the faster is the line's step.  Tokens/s, per-kernel
    times and algorithmic GB/s."""
    if splits:
        w = w.scaled(num_splits=splits)
    c = W.make_sparse_case(w, device=dev)
    kv = sdv.PagedKV(c.k_pool, c.v_pool, c.k_scale, c.v_scale)
    mq = w.max_qo()
    rows_cap = w.batch * mq
    q = torch.zeros((rows_cap, w.num_q_heads, w.head_dim), dtype=c.q.dtype, device=dev)
    q[:c.q.shape[0]] = c.q
    scores = torch.empty((rows_cap, w.num_kv_heads, w.max_pages()), dtype=torch.float32, device=dev)
    idx = torch.empty((rows_cap, w.num_kv_heads, w.top_k), dtype=torch.int32, device=dev)
    out = torch.empty((rows_cap, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    ws = sdv.alloc_workspace(rows_cap, w.num_q_heads, w.head_dim, w.num_splits, dev, op="sparse")

    def k_proxy():
        sdv.proxy_page_scores(q, c.qo_indptr, c.kv_len, kv, c.block_table, max_qo_len=mq,
                              scores=scores)

    def k_select():
        sdv.verify_attention_sparse_select(q, c.qo_indptr, c.kv_len, kv, c.block_table, scores,
                                           max_qo_len=mq, top_k=w.top_k,
                                           softmax_scale=c.softmax_scale,
                                           num_splits=w.num_splits, workspace=ws, out=out,
                                           family=fam)

    def k_topk():
        sdv.ladder_topk_pages(scores, c.qo_indptr, c.kv_len, max_qo_len=mq, top_k=w.top_k,
                              topk_idx=idx)

    def k_sparse():
        sdv.verify_attention_sparse(q, c.qo_indptr, c.kv_len, kv, c.block_table, idx,
                                    max_qo_len=mq, softmax_scale=c.softmax_scale,
                                    num_splits=w.num_splits, workspace=ws, out=out, family=fam)

    paths = {
        "fused": [("proxy_page_scores", k_proxy), ("verify_attention_sparse_select", k_select)],
        "three_launch": [("proxy_page_scores", k_proxy), ("ladder_topk_pages", k_topk),
                         ("verify_attention_sparse", k_sparse)]}
    timed = {p: time_steps(f, args.steps, args.warmup, torch, flush) for p, f in paths.items()}
    # the selection, written out once after timing, sizes the algorithmic bytes
    k_topk()
    torch.cuda.synchronize()
    ab = sparse_algorithmic_bytes(c, idx.cpu().numpy())
    keys = {"proxy_page_scores": "proxy", "verify_attention_sparse_select": "select",
            "ladder_topk_pages": "topk", "verify_attention_sparse": "sparse"}
    tokens = c.lengths.total_q
    lines = {}
    for p, (ms, per, _) in timed.items():
        kern = {}
        for name in per:
            key = keys[name]
            gbs = ab[key] / (per[name]["avg_us"] * 1e-6) / 1e9
            kern[name] = {**per[name], "algorithmic_bytes": ab[key], "GB_s": gbs,
                          "frac_of_peak": gbs / HBM_PEAK_GBS,
                          "traffic": load_traffic(name, w.name, source_hash(*KERNEL_SOURCES[name]))}
        path = sum(ab[keys[name]] for name in per)
        dom = max(kern, key=lambda k: kern[k]["avg_us"])
        lines[p] = {"value": tokens / (ms * 1e-3), "ms_per_step": ms,
                    "path_algorithmic_bytes": path, "gb_per_s": path / (ms * 1e-3) / 1e9,
                    "frac_of_peak": path / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "roofline": {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["GB_s"],
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": kern[dom]["GB_s"] / HBM_PEAK_GBS,
                                 "traffic": kern[dom]["traffic"]},
                    "kernels": kern}
    best = min(lines, key=lambda p: lines[p]["ms_per_step"])
    res = {"step": best, **{k: v for k, v in lines[best].items()}, "unit": "verify tokens/s",
           "verify_tokens": tokens, "kv_tokens": int(c.lengths.kv.sum()),
           "num_splits": w.num_splits, "paths": {p: {"ms_per_step": v["ms_per_step"],
                                                     "kernels": v["kernels"]}
                                                 for p, v in lines.items()}}
    del c, kv, q, scores, idx, out, ws
    return res


def dense_config_line(torch, sdv, W, w, dev, args, flush, fam, splits=None):
    """The dense draft-layer step through the P32 view (page indices computed in the
    attention launch, + the split-KV combine) on workload w."""
    splits = splits or w.num_splits
    d = W.make_dense_case(w, device=dev)
    mq = w.max_qo()
    rows_cap = w.batch * mq
    q = torch.zeros((rows_cap, w.num_q_heads, w.head_dim), dtype=d.q.dtype, device=dev)
    q[:d.q.shape[0]] = d.q
    out = torch.empty((rows_cap, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    ws = sdv.alloc_workspace(rows_cap, w.num_q_heads, w.head_dim, splits, dev)
    view, _ = sdv.kv_subpage_view_init(
        d.pool[w.root_page], d.block_table, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
        slot_stride=w.slot_stride, num_slots=d.num_slots, k_scale=d.k_scale, v_scale=d.v_scale,
        pool_index_scale=w.pool_index_scale, stage_offsets=False)

    def k_dview():
        sdv.verify_attention_dense_view(q, d.qo_indptr, d.kv_len, view, d.block_table,
                                        max_qo_len=mq, softmax_scale=d.softmax_scale,
                                        num_splits=splits, workspace=ws, out=out, family=fam)

    name = "verify_attention_dense_view"
    ms, per, _ = time_steps([(name, k_dview)], args.steps, args.warmup, torch, flush)
    db = dense_algorithmic_bytes(d)
    gbs = db / (per[name]["avg_us"] * 1e-6) / 1e9
    tokens = d.lengths.total_q
    res = {"value": tokens / (ms * 1e-3), "unit": "verify tokens/s", "ms_per_step": ms,
           "verify_tokens": tokens, "kv_tokens": int(d.lengths.kv.sum()), "num_splits": splits,
           "algorithmic_bytes": db, "kernels": per,
           "roofline": {"bound": "hbm", "kernel": name, "achieved": gbs, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                        "traffic": load_traffic(name, w.name, source_hash(*KERNEL_SOURCES[name]))}}
    del d, q, out, ws, view
    return res


def calibrate_copy(torch, mib=1024, reps=3):
    """A plain device copy of known size, for scaling the memory counters."""
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": mib << 20, "copy_bytes_written": mib << 20,
                      "reps": reps}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the verify path "
              "here is a single-GPU kernel library with no cross-GPU step.", file=sys.stderr)
        sys.exit(2)
    oracle_pool = None
    headline = args.only is None or "sparse" in args.only.split(",")
    if not args.no_cpu_baseline and not args.calibrate_copy and headline:
        oracle_pool = start_oracle_pool()
    import torch

    import speculative_decode_verify_p128_amd as sdv
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    fam = args.family
    only = set(args.only.split(",")) if args.only else None

    def want(section, disabled=False):
        return (section in only) if only is not None else not disabled

    flush = None
    if not args.warm:
        flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

        def flush():
            sdv.fill_u32(flush_buf, 0x5A5A5A5A)

    # ---- sparse target-layer path (the headline workload) ----
    # (skipped only when --only names sections without "sparse": profiling runs of other
    # sections, whose JSON line then carries just those sections)
    c = None
    if only is None or "sparse" in only:
        w = W.SPARSE_BF16
        splits = args.splits or w.num_splits
        c = W.make_sparse_case(w, device=dev)
        kv = sdv.PagedKV(c.k_pool, c.v_pool, c.k_scale, c.v_scale)
        rows_cap = w.batch * w.max_qo()
        scores = torch.empty((rows_cap, w.num_kv_heads, w.max_pages()), dtype=torch.float32, device=dev)
        idx = torch.empty((rows_cap, w.num_kv_heads, w.top_k), dtype=torch.int32, device=dev)
        out = torch.empty((rows_cap, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        ws = sdv.alloc_workspace(rows_cap, w.num_q_heads, w.head_dim, splits, dev, op="sparse")
        mq = w.max_qo()

        def k_proxy():
            sdv.proxy_page_scores(c.q, c.qo_indptr, c.kv_len, kv, c.block_table, max_qo_len=mq,
                                  scores=scores)

        def k_topk():
            sdv.ladder_topk_pages(scores, c.qo_indptr, c.kv_len, max_qo_len=mq, top_k=w.top_k,
                                  topk_idx=idx)

        def k_sparse():
            sdv.verify_attention_sparse(c.q, c.qo_indptr, c.kv_len, kv, c.block_table, idx,
                                        max_qo_len=mq, softmax_scale=c.softmax_scale,
                                        num_splits=splits, workspace=ws, out=out, family=fam)

        def k_select():
            sdv.verify_attention_sparse_select(c.q, c.qo_indptr, c.kv_len, kv, c.block_table, scores,
                                               max_qo_len=mq, top_k=w.top_k,
                                               softmax_scale=c.softmax_scale, num_splits=splits,
                                               workspace=ws, out=out, family=fam)

        fns = [("proxy_page_scores", k_proxy), ("verify_attention_sparse_select", k_select)]
        launch_stats = {}
        eager_ms, per, wall = time_steps(fns, args.steps, args.warmup, torch, flush, launch_stats)
        ms = eager_ms
        if args.graph:
            # the step as one HIP graph (the path is capture-safe: no allocation, no host
            # synchronisation, lengths read on the device); its outputs must equal the eager ones
            ref_out = out.clone()
            ms = time_graph(fns, args.steps, args.warmup, torch, flush)
            if not torch.equal(out.view(torch.int16), ref_out.view(torch.int16)):
                raise RuntimeError("graph replay of the sparse path differs from its eager run")
            del ref_out
        # the selection the fused launch made (written out here, after timing) sizes the
        # algorithmic bytes; the two-launch path must reach the same output
        fused_out = out.clone()
        k_proxy()
        k_topk()
        k_sparse()
        torch.cuda.synchronize()
        if not torch.equal(out.view(torch.int16), fused_out.view(torch.int16)):
            raise RuntimeError("in-kernel selection and standalone top-k give different outputs")
        del fused_out
        tokens = c.lengths.total_q
        idx_np = idx.cpu().numpy()
        ab = sparse_algorithmic_bytes(c, idx_np)
        path_bytes = ab["proxy"] + ab["select"]
        kern = {}
        for name, key in (("proxy_page_scores", "proxy"), ("verify_attention_sparse_select", "select")):
            gbs = ab[key] / (per[name]["avg_us"] * 1e-6) / 1e9
            kern[name] = {**per[name], "algorithmic_bytes": ab[key], "GB_s": gbs,
                          "frac_of_peak": gbs / HBM_PEAK_GBS}
        unfused = None
        if want("unfused", args.no_unfused):
            ufns = [("proxy_page_scores", k_proxy), ("ladder_topk_pages", k_topk),
                    ("verify_attention_sparse", k_sparse)]
            u_ms, u_per, _ = time_steps(ufns, args.steps, args.warmup, torch, flush)
            unfused = {"ms_per_step": u_ms, "kernels": {}}
            for name, key in (("proxy_page_scores", "proxy"), ("ladder_topk_pages", "topk"),
                              ("verify_attention_sparse", "sparse")):
                gbs = ab[key] / (u_per[name]["avg_us"] * 1e-6) / 1e9
                unfused["kernels"][name] = {**u_per[name], "algorithmic_bytes": ab[key], "GB_s": gbs,
                                            "frac_of_peak": gbs / HBM_PEAK_GBS}
        dom = max(kern, key=lambda k: kern[k]["avg_us"])
        traffic = load_traffic(dom, w.name, source_hash(*KERNEL_SOURCES[dom]))
        path_gbs = path_bytes / (ms * 1e-3) / 1e9
        result = {
            "metric": METRIC,
            "value": tokens / (ms * 1e-3),
            "unit": "verify tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": ms,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic (seeded, generated on the GPU)",
            "config": {"workload": "sparse_bf16: block-sparse target-layer verify, batch 64, "
                                   "qo_len 4, 16 q / 4 kv heads, head_dim 128, kv_len U[4096, 32768], "
                                   "128-token pages, top-k 16",
                       "batch": w.batch, "qo_len": 4, "num_q_heads": w.num_q_heads,
                       "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "top_k": w.top_k,
                       "num_splits": splits, "seed": W.seed_for(w), "verify_tokens": tokens,
                       "kv_tokens": int(c.lengths.kv.sum())},
            "gb_per_s": path_gbs,
            "frac_of_peak": path_gbs / HBM_PEAK_GBS,
            "path_algorithmic_bytes": path_bytes,
            "roofline": {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["GB_s"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": kern[dom]["GB_s"] / HBM_PEAK_GBS,
                         "traffic": traffic},
            "kernels": kern,
            "launch": ("one HIP graph replay per step (proxy, selection + attention); the per-kernel "
                       "times in kernels come from an eager pass with events around every launch"
                       if args.graph else "eager: one launch per kernel"),
            "eager_ms_per_step": eager_ms,
            "ms_per_step_with_launch_events": launch_stats.get("ms_per_step_with_launch_events"),
            "unfused": unfused,
            "sparse_row_expanded_kv_bytes": ab["sparse_row_expanded_kv"],
            "wall_s_timed": wall,
            "cache": ("warm: consecutive steps, no eviction" if args.warm else
                      "cold: a 1 GiB fill before every step (untimed) evicts L2 and the Infinity Cache"),
        }
        if not args.no_probe:
            # what the two kernels' own access patterns attain: their gather lists streamed
            # once by the unit-list probe, cold
            pu, su = sparse_gather_units(c, idx_np, torch, dev)
            att = {"proxy_page_scores": units_read_gbs(torch, sdv, dev, [(c.k_pool, pu, 16384)], flush),
                   "verify_attention_sparse_select": units_read_gbs(
                       torch, sdv, dev, [(c.k_pool, su, 16384), (c.v_pool, su, 16384)], flush)}
            for name, gbs_att in att.items():
                kern[name]["attainable_read_GB_s"] = gbs_att
                kern[name]["frac_of_attainable"] = kern[name]["GB_s"] / gbs_att
            del pu, su
        del scores, ws

    else:
        result = {"metric": METRIC, "sections_only": sorted(only)}

    # ---- dense draft-layer path ----
    if want("dense", args.no_dense):
        wd = W.DENSE_BF16
        dsplits = args.dense_splits or wd.num_splits
        d = W.make_dense_case(wd, device=dev)
        rows_d = wd.batch * wd.max_qo()
        outd = torch.empty((rows_d, wd.num_q_heads, wd.head_dim), dtype=torch.bfloat16, device=dev)
        wsd = sdv.alloc_workspace(rows_d, wd.num_q_heads, wd.head_dim, dsplits, dev)
        offs = torch.empty((wd.batch, 2, 4 * wd.max_pages()), dtype=torch.int32, device=dev)
        holder = {}
        view_only, _ = sdv.kv_subpage_view_init(
            d.pool[wd.root_page], d.block_table, num_kv_heads=wd.num_kv_heads,
            head_dim=wd.head_dim, slot_stride=wd.slot_stride, num_slots=d.num_slots,
            pool_index_scale=wd.pool_index_scale, stage_offsets=False)

        def k_dview():
            sdv.verify_attention_dense_view(d.q, d.qo_indptr, d.kv_len, view_only, d.block_table,
                                            max_qo_len=wd.max_qo(), softmax_scale=d.softmax_scale,
                                            num_splits=dsplits, workspace=wsd, out=outd,
                                            family=fam)

        def k_view():
            holder["view"], _ = sdv.kv_subpage_view_init(
                d.pool[wd.root_page], d.block_table, num_kv_heads=wd.num_kv_heads,
                head_dim=wd.head_dim, slot_stride=wd.slot_stride, num_slots=d.num_slots,
                pool_index_scale=wd.pool_index_scale, sub_offsets=offs)

        def k_dense():
            sdv.verify_attention_dense(d.q, d.qo_indptr, d.kv_len, holder["view"], offs,
                                       max_qo_len=wd.max_qo(), softmax_scale=d.softmax_scale,
                                       num_splits=dsplits, workspace=wsd, out=outd, family=fam)

        # the step: the view's page indices computed inside the attention launch
        msd, perd, _ = time_steps([("verify_attention_dense_view", k_dview)],
                                  args.steps, args.warmup, torch, flush)
        # the two-call path (view offsets, then attention over them) must give the same bits
        fused_out = outd.clone()
        k_view()
        k_dense()
        torch.cuda.synchronize()
        if not torch.equal(outd.view(torch.int16), fused_out.view(torch.int16)):
            raise RuntimeError("dense view in the attention launch and the two-call path differ")
        del fused_out
        db = dense_algorithmic_bytes(d)
        gbs = db / (perd["verify_attention_dense_view"]["avg_us"] * 1e-6) / 1e9
        result["dense"] = {
            "workload": "dense_bf16: draft-layer verify through the P32 view, batch 32, qo_len 4, "
                        "64 q / 4 kv heads, head_dim 128, kv_len U[1024, 8192], slot stride 8",
            "value": d.lengths.total_q / (msd * 1e-3), "unit": "verify tokens/s",
            "ms_per_step": msd, "num_splits": dsplits, "algorithmic_bytes": db,
            "kernels": perd,
            "roofline": {"bound": "hbm", "kernel": "verify_attention_dense_view", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": load_traffic("verify_attention_dense_view", wd.name,
                                                 source_hash(*KERNEL_SOURCES["verify_attention_dense_view"]))},
        }
        if not args.no_probe:
            # what the call's own access pattern attains: the K and V runs (8 KiB each) of
            # every block it reads, streamed once by the unit-list probe, cold
            k_view()
            torch.cuda.synchronize()
            o_ = offs.cpu().numpy()
            unit = wd.head_dim * 2 * 32
            root = d.pool[wd.root_page]
            shift = root.data_ptr() - d.pool.data_ptr()
            assert shift % unit == 0
            lst = []
            for r_ in range(wd.batch):
                nb_ = (int(d.lengths.kv[r_]) + 31) // 32
                for h_ in range(wd.num_kv_heads):
                    lst.append(o_[r_, 0, :nb_].astype(np.int64) * wd.num_kv_heads + h_)
                    lst.append(o_[r_, 1, :nb_].astype(np.int64) * wd.num_kv_heads + h_)
            units_d = torch.from_numpy(np.concatenate(lst) + shift // unit).to(dev)
            result["dense"]["attainable_read_GB_s"] = units_read_gbs(
                torch, sdv, dev, [(d.pool, units_d, unit)], flush)
            result["dense"]["frac_of_attainable"] = gbs / result["dense"]["attainable_read_GB_s"]
            del units_d
        if args.dense_two_call:
            ms2, per2, _ = time_steps([("kv_subpage_view_init", k_view),
                                       ("verify_attention_dense", k_dense)],
                                      args.steps, args.warmup, torch, flush)
            result["dense"]["two_call"] = {"ms_per_step": ms2, "kernels": per2,
                                           "algorithmic_bytes": dense_algorithmic_bytes(d, True)}
        del d, outd, wsd

    # ---- long-context sparse verify with fp8 K/V, 16-way split-KV ----
    if want("long_fp8", args.no_extra_configs):
        result["long_fp8"] = {
            "workload": "long_fp8: sparse verify, batch 8, qo_len 4, 16 q / 4 kv heads, head_dim "
                        "128, kv_len 131072, fp8 e4m3 K/V with per-tensor scales, bf16 Q, top-k "
                        "64, 16 splits",
            **sparse_config_line(torch, sdv, W, W.LONG_FP8, dev, args, flush, fam,
                                 args.long_splits)}

    # ---- ragged mixed batch through both paths ----
    if want("ragged", args.no_extra_configs):
        wr = W.RAGGED_MIXED
        result["ragged_mixed"] = {
            "workload": "ragged_mixed: batch 256, qo_len 1..8, kv_len log-normal (median 2048, "
                        "clipped [64, 65536]) with page-crossing rows, 16 q / 4 kv heads, "
                        "head_dim 128, bf16, top-k 16 clamped",
            # split counts: the fastest measured for each path (sparse 1-4, dense 2-16: 6 and 8
            # within 1 us, 4 about 8 us slower)
            "sparse": sparse_config_line(torch, sdv, W, wr, dev, args, flush, fam,
                                         args.ragged_splits or 1),
            "dense": dense_config_line(torch, sdv, W, wr, dev, args, flush, fam,
                                       args.ragged_dense_splits or 6)}

    # ---- target dense layers: ladder attention over ordinary head-major P128 pages ----
    if want("paged", args.no_paged):
        wp = W.PAGED_BF16
        psplits = args.paged_splits or wp.num_splits
        pc = W.make_sparse_case(wp, device=dev)
        pkv = sdv.PagedKV(pc.k_pool, pc.v_pool, pc.k_scale, pc.v_scale)
        rows_p = wp.batch * wp.max_qo()
        outp = torch.empty((rows_p, wp.num_q_heads, wp.head_dim), dtype=torch.bfloat16, device=dev)
        wsp = sdv.alloc_workspace(rows_p, wp.num_q_heads, wp.head_dim, psplits, dev, op="paged")

        def k_paged():
            sdv.verify_attention_paged(pc.q, pc.qo_indptr, pc.kv_len, pkv, pc.block_table,
                                       max_qo_len=wp.max_qo(), softmax_scale=pc.softmax_scale,
                                       num_splits=psplits, workspace=wsp, out=outp, family=fam)

        msp, perp, _ = time_steps([("verify_attention_paged", k_paged)], args.steps, args.warmup,
                                  torch, flush)
        pb = paged_algorithmic_bytes(pc)
        gbs = pb / (perp["verify_attention_paged"]["avg_us"] * 1e-6) / 1e9
        result["paged"] = {
            "workload": "paged_bf16: target dense-layer verify over head-major P128 pages, batch 64, "
                        "qo_len 4, 16 q / 4 kv heads, head_dim 128, kv_len U[4096, 32768]",
            "value": pc.lengths.total_q / (msp * 1e-3), "unit": "verify tokens/s",
            "ms_per_step": msp, "num_splits": psplits, "algorithmic_bytes": pb,
            "kernels": perp,
            "roofline": {"bound": "hbm", "kernel": "verify_attention_paged", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": load_traffic("verify_attention_paged", wp.name,
                                                 source_hash(*KERNEL_SOURCES["verify_attention_paged"]))},
        }
        del pc, pkv, outp, wsp

    # ---- ladder KV slot staging of the verify tokens (the step before the path) ----
    if want("staging", args.no_paged):
        ws_ = W.PAGED_BF16
        sc = W.make_sparse_case(ws_, device=dev)
        rows_s = sc.lengths.total_q
        g = torch.Generator(device=dev).manual_seed(W.seed_for(ws_))
        kn = torch.randn((rows_s, ws_.num_kv_heads, ws_.head_dim), generator=g,
                         device=dev).to(torch.bfloat16)
        vn = torch.randn_like(kn)
        skv = sdv.PagedKV(sc.k_pool, sc.v_pool)

        def k_stage():
            sdv.stage_verify_kv_paged(kn, vn, sc.qo_indptr, sc.kv_len, skv, sc.block_table,
                                      max_qo_len=ws_.max_qo())

        mss, pers, _ = time_steps([("stage_verify_kv_paged", k_stage)], args.steps, args.warmup,
                                  torch, flush)
        sb = 2 * 2 * rows_s * ws_.num_kv_heads * ws_.head_dim * 2   # K and V rows, read + write
        result["staging"] = {
            "workload": "paged_bf16 verify tokens: 256 rows x 4 kv heads x 128 channels of K and "
                        "V into head-major P128 pages",
            "kernels": pers, "algorithmic_bytes": sb,
            "GB_s": sb / (pers["stage_verify_kv_paged"]["avg_us"] * 1e-6) / 1e9,
            "bound": "latency (one small launch)",
        }
        del sc, skv, kn, vn

    # ---- grouped head-major head-slice transfer of the draft layer (two TP ranks -> one) ----
    if want("transfer", args.no_dense):
        wt = W.DENSE_BF16
        dc = W.make_dense_case(wt, device=dev)
        H, per = wt.num_kv_heads, wt.num_kv_heads // 2
        pages = [s_ * wt.slot_stride + wt.root_page for s_ in range(dc.num_slots)]
        pages = np.array(pages + [p_ + 1 for p_ in pages])
        e_ = dc.pool.element_size()
        senders = [dc.pool[:, :, r_ * per:(r_ + 1) * per].contiguous() for r_ in range(2)]
        recv = torch.zeros_like(dc.pool)
        descs = [torch.from_numpy(sdv.hnd_head_slice_descriptors(
            token_groups=4, src_heads=per, src_head_begin=0, dst_heads=H, dst_head_begin=r_ * per,
            num_heads=per, head_dim=wt.head_dim, kv_dtype=dc.pool.dtype,
            src_page_offsets=pages * (4 * per * 32 * wt.head_dim * e_),
            dst_page_offsets=pages * (4 * H * 32 * wt.head_dim * e_))).to(dev) for r_ in range(2)]

        def k_transfer():
            for r_ in range(2):
                sdv.copy_descriptors(senders[r_], recv, descs[r_])

        mst, pert, _ = time_steps([("copy_descriptors", k_transfer)], args.steps, args.warmup,
                                  torch, flush)
        tb = 2 * len(pages) * 4 * H * 32 * wt.head_dim * e_          # read + written
        gbs = tb / (pert["copy_descriptors"]["avg_us"] * 1e-6) / 1e9
        result["transfer"] = {
            "workload": "dense_bf16 draft layer (K and V of every slot, grouped head-major P128 "
                        "pages) from two 2-head ranks into one 4-head pool, one descriptor per "
                        "(page, K/V, token group)",
            "kernels": pert, "bytes_read_and_written": tb,
            "roofline": {"bound": "hbm", "kernel": "copy_descriptors", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": load_traffic("copy_descriptors", wt.name,
                                                 source_hash(*KERNEL_SOURCES["copy_descriptors"]))},
        }
        del dc, senders, recv, descs

    # ---- greedy acceptance after the verify step (target argmax vs draft tokens) ----
    if want("accept", args.no_paged):
        wa = W.SPARSE_BF16
        ac = W.make_accept_case(wa, ACCEPT_VOCAB, device=dev)
        acc_outs = (torch.empty(wa.batch * wa.max_qo(), dtype=torch.int32, device=dev),
                    torch.empty(wa.batch, dtype=torch.int32, device=dev),
                    torch.empty((wa.batch, wa.max_qo()), dtype=torch.int32, device=dev),
                    torch.empty(wa.batch, dtype=torch.int32, device=dev))
        acc_ws = torch.empty(sdv.greedy_accept_workspace_bytes(wa.batch, wa.max_qo(), ACCEPT_VOCAB,
                                                               torch.bfloat16),
                             dtype=torch.uint8, device=dev)

        def k_accept():
            sdv.greedy_accept(ac.logits, ac.tokens, ac.qo_indptr, ac.kv_len, max_qo_len=wa.max_qo(),
                              outs=acc_outs, workspace=acc_ws)

        msa, pera, _ = time_steps([("greedy_accept", k_accept)], args.steps, args.warmup, torch,
                                  flush)
        ab_ = ac.lengths.total_q * ACCEPT_VOCAB * 2 + ac.lengths.total_q * 4 * 2
        gbs = ab_ / (pera["greedy_accept"]["avg_us"] * 1e-6) / 1e9
        result["accept"] = {
            "workload": f"sparse_bf16 verify rows: 256 rows of {ACCEPT_VOCAB} bf16 logits (synthetic "
                        "vocabulary size), greedy argmax and accepted-prefix per request",
            "kernels": pera, "algorithmic_bytes": ab_,
            "roofline": {"bound": "hbm", "kernel": "greedy_accept", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": load_traffic("greedy_accept", wa.name,
                                                 source_hash(*KERNEL_SOURCES["greedy_accept"]))},
        }
        del ac

    if not args.no_probe:
        result["attainable_read_GB_s"] = attainable_read_gbs(torch, sdv, dev)
    if not args.no_cpu_baseline and c is not None:
        c_cpu = W.SparseCase(**{**c.__dict__})
        result["cpu_baseline"] = cpu_baseline(c_cpu, args.cpu_sample)
        result["cpu_baseline"]["cpu_model"] = host_cpu_model()
        pool, procs = oracle_pool
        try:
            result["cpu_baseline"]["all_cores"] = cpu_baseline_all_cores(c_cpu, args.cpu_sample,
                                                                         pool, procs)
        finally:
            pool.close()
            pool.join()
    else:
        result["cpu_baseline"] = None
        if oracle_pool is not None:
            oracle_pool[0].close()
            oracle_pool[0].join()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
