"""GPU parity of ladder KV slot staging against the oracle: whole pools compared bit for
bit after staging (head-major pages and the P32 view; bf16, fp8 and fp32 storage,
page-crossing ladders), the overlap-correction re-stage followed by attention over the
result, device error flags, and the full benchmark size checked by properties."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_p128_amd as sdv
import workloads as W
from oracle.staging import stage_paged, stage_view
from workloads import raw_numpy

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _parity import DEV, PagedRun, out_numpy, paged_oracle, tol_ok

STAGE_HND = [
    W.PAGED_BF16.scaled(name="stage_bf16", batch=5, kv=("uniform", 4, 600), kv_capacity=640),
    W.LONG_FP8.scaled(name="stage_fp8", batch=3, kv=("uniform", 120, 700), kv_capacity=768),
    W.TINY_FP32,
    W.RAGGED_MIXED.scaled(name="stage_ragged", batch=16, kv=("lognormal", 300, 1.0, 1, 2000, 0.25),
                          kv_capacity=2048),
]
STAGE_VIEW = [
    W.DENSE_BF16.scaled(name="stage_view_bf16", batch=4, kv=("uniform", 4, 900), kv_capacity=1024),
    W.TINY_FP32,
]


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


def _new_rows(rows, H, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((rows, H, d), generator=g)
    v = torch.randn((rows, H, d), generator=g)
    if dtype == torch.float8_e4m3fn:
        return k.to(dtype), v.to(dtype)
    return k.to(dtype), v.to(dtype)


def _raw(t):
    return raw_numpy(t.cpu())


@pytest.mark.parametrize("w", STAGE_HND, ids=lambda w: w.name)
def test_stage_paged_bit_exact(w):
    c = W.make_sparse_case(w)
    rows = w.batch * w.max_qo()
    kn, vn = _new_rows(rows, w.num_kv_heads, w.head_dim, c.k_pool.dtype, 11)
    ref_k, ref_v = stage_paged(_raw(c.k_pool), _raw(c.v_pool), _raw(kn), _raw(vn),
                               c.qo_indptr.numpy(), c.lengths.kv, c.block_table.numpy())
    kp, vp = c.k_pool.to(DEV), c.v_pool.to(DEV)
    kv = sdv.PagedKV(kp, vp, c.k_scale, c.v_scale)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    sdv.stage_verify_kv_paged(kn.to(DEV), vn.to(DEV), c.qo_indptr.to(DEV), c.kv_len.to(DEV), kv,
                              c.block_table.to(DEV), max_qo_len=w.max_qo(), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(_raw(kp), ref_k) and np.array_equal(_raw(vp), ref_v)


@pytest.mark.parametrize("w", STAGE_VIEW, ids=lambda w: w.name)
def test_stage_view_bit_exact(w):
    c = W.make_dense_case(w)
    rows = w.batch * w.max_qo()
    kn, vn = _new_rows(rows, w.num_kv_heads, w.head_dim, c.pool.dtype, 12)
    page_elems = 4 * w.num_kv_heads * 32 * w.head_dim
    ref = stage_view(_raw(c.pool).reshape(-1), w.root_page * page_elems, _raw(kn), _raw(vn),
                     c.qo_indptr.numpy(), c.lengths.kv, c.block_table.numpy(), w.slot_stride,
                     w.num_kv_heads, w.head_dim)
    pool = c.pool.to(DEV)
    bt = c.block_table.to(DEV)
    view, offs = sdv.kv_subpage_view_init(pool[w.root_page], bt, num_kv_heads=w.num_kv_heads,
                                          head_dim=w.head_dim, slot_stride=w.slot_stride,
                                          num_slots=c.num_slots, pool_index_scale=w.pool_index_scale)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    sdv.stage_verify_kv_view(kn.to(DEV), vn.to(DEV), c.qo_indptr.to(DEV), c.kv_len.to(DEV), view,
                             offs, max_qo_len=w.max_qo(), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(_raw(pool).reshape(-1), ref)


def test_overlap_correction_restage_then_attention():
    """Step A stages 4 tokens per request; a correction shortens request 1 across a page
    boundary (131 -> 128 positions); step B stages the next 4 tokens at the corrected
    positions.  The pools match the oracle bit for bit and attention over them matches
    the oracle's attention."""
    w = W.PAGED_BF16.scaled(name="restage", batch=3, kv=("fixed", 384), kv_capacity=512)
    c = W.make_sparse_case(w)
    kv_a = np.array([200, 131, 300])
    kv_b = np.array([204, 132, 304])
    ind = c.qo_indptr.numpy()
    kn_a, vn_a = _new_rows(12, w.num_kv_heads, w.head_dim, torch.bfloat16, 21)
    kn_b, vn_b = _new_rows(12, w.num_kv_heads, w.head_dim, torch.bfloat16, 22)
    bt = c.block_table.numpy()
    rk, rv = stage_paged(_raw(c.k_pool), _raw(c.v_pool), _raw(kn_a), _raw(vn_a), ind, kv_a, bt)
    rk, rv = stage_paged(rk, rv, _raw(kn_b), _raw(vn_b), ind, kv_b, bt)
    kp, vp = c.k_pool.to(DEV), c.v_pool.to(DEV)
    kvd = sdv.PagedKV(kp, vp)
    qo_d, bt_d = c.qo_indptr.to(DEV), c.block_table.to(DEV)
    for kn, vn, lens in ((kn_a, vn_a, kv_a), (kn_b, vn_b, kv_b)):
        sdv.stage_verify_kv_paged(kn.to(DEV), vn.to(DEV), qo_d,
                                  torch.tensor(lens, dtype=torch.int32, device=DEV), kvd, bt_d,
                                  max_qo_len=4)
    torch.cuda.synchronize()
    assert np.array_equal(_raw(kp), rk) and np.array_equal(_raw(vp), rv)
    # attention over the re-staged cache
    c.k_pool, c.v_pool = kp.cpu(), vp.cpu()
    c.lengths.kv[:] = kv_b
    c.kv_len[:] = torch.tensor(kv_b, dtype=torch.int32)
    run = PagedRun(c)
    out = run.attend_paged()
    torch.cuda.synchronize()
    ok, worst = tol_ok(out_numpy(out[:run.n]), paged_oracle(c), "bf16")
    assert ok, worst


def test_stage_flags():
    w = STAGE_HND[0]
    c = W.make_sparse_case(w)
    kn, vn = _new_rows(w.batch * w.max_qo(), w.num_kv_heads, w.head_dim, torch.bfloat16, 13)
    kv = sdv.PagedKV(c.k_pool.to(DEV), c.v_pool.to(DEV))
    bt = c.block_table.clone()
    bt[0, :] = c.k_pool.shape[0] + 3                   # request 0: pages out of range
    lens = c.kv_len.clone()
    lens[1] = w.max_pages() * 128 + 1                   # request 1: beyond capacity
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    sdv.stage_verify_kv_paged(kn.to(DEV), vn.to(DEV), c.qo_indptr.to(DEV), lens.to(DEV), kv,
                              bt.to(DEV), max_qo_len=w.max_qo(), dev_err=err)
    torch.cuda.synchronize()
    e = int(err.item())
    assert e & sdv._lib.DEVERR_PAGE_RANGE and e & sdv._lib.DEVERR_KV_CAPACITY


def test_stage_full_size_properties():
    """At the benchmark size: every staged position holds its new row and exactly the
    staged elements changed."""
    w = W.PAGED_BF16
    c = W.make_sparse_case(w, device=DEV)
    rows = w.batch * w.max_qo()
    g = torch.Generator(device=DEV).manual_seed(31)
    kn = torch.randn((rows, w.num_kv_heads, w.head_dim), generator=g, device=DEV).to(torch.bfloat16)
    vn = torch.randn((rows, w.num_kv_heads, w.head_dim), generator=g, device=DEV).to(torch.bfloat16)
    k0, v0 = c.k_pool.clone(), c.v_pool.clone()
    kv = sdv.PagedKV(c.k_pool, c.v_pool)
    sdv.stage_verify_kv_paged(kn, vn, c.qo_indptr, c.kv_len, kv, c.block_table, max_qo_len=4)
    torch.cuda.synchronize()
    ind = c.qo_indptr.cpu().numpy()
    lens = c.lengths.kv
    bt = c.block_table.cpu().numpy()
    pages, slots, src = [], [], []
    for r in range(w.batch):
        for t in range(ind[r + 1] - ind[r]):
            j = int(lens[r]) - (ind[r + 1] - ind[r]) + t
            pages.append(bt[r, j // 128]); slots.append(j % 128); src.append(ind[r] + t)
    pages = torch.tensor(pages, device=DEV)
    slots = torch.tensor(slots, device=DEV)
    src = torch.tensor(src, device=DEV)
    for pool, old, new in ((c.k_pool, k0, kn), (c.v_pool, v0, vn)):
        got = pool[pages, :, slots, :]                          # [rows, Hkv, d]
        assert torch.equal(got.view(torch.int16), new[src].view(torch.int16))
        changed = int((pool.view(torch.int16) != old.view(torch.int16)).sum().item())
        expect = int((old[pages, :, slots, :].view(torch.int16) != new[src].view(torch.int16)).sum().item())
        assert changed == expect
