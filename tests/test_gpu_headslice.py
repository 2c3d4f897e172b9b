"""GPU: the grouped head-major head-slice transfer of a draft layer from two tensor-
parallel context ranks (two KV heads each) to a four-head generation pool, through the
library's mapper and its device copy engine.  Every logical (K/V, head) tensor is
reconstructed and compared by SHA-256 with the source (the pages' transfer proof); the
one-slice-per-page mapping is wrong after the first token group; attention through the
P32 view over the received pool matches the oracle on the original."""
import hashlib

import numpy as np
import pytest
import torch

import speculative_decode_verify_p128_amd as sdv
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _parity import DEV, DenseRun, dense_oracle, out_numpy, tol_ok

CASE = W.DENSE_BF16.scaled(name="transfer", batch=3, kv=("uniform", 100, 900), kv_capacity=1024)


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


def _draft_pages(w, num_slots):
    ks = [s * w.slot_stride + w.root_page for s in range(num_slots)]
    return ks + [k + 1 for k in ks]


def _logical_digests(pool, pages):
    """SHA-256 of each logical (K/V, head) tensor [slots, 128 tokens, d] of the layer."""
    n = len(pages) // 2
    out = {}
    for kind, sel in (("K", pages[:n]), ("V", pages[n:])):
        x = pool[torch.tensor(sel, device=pool.device)]            # [slots, 4, H, 32, d]
        H = x.shape[2]
        for h in range(H):
            t = x[:, :, h].reshape(len(sel), 128, -1).contiguous().cpu()
            out[(kind, h)] = hashlib.sha256(t.view(torch.int16).numpy().tobytes()).hexdigest()
    return out


def _transfer(c, groups, dev_err=None):
    w = c.w
    pool = c.pool.to(DEV)
    pages = _draft_pages(w, c.num_slots)
    recv = pool.clone()
    recv[torch.tensor(pages, device=DEV)] = 0
    H, per = w.num_kv_heads, w.num_kv_heads // 2
    e = pool.element_size()
    recv_page_b = 4 * H * 32 * w.head_dim * e
    send_page_b = 4 * per * 32 * w.head_dim * e
    for rank in range(2):
        sender = pool[:, :, rank * per:(rank + 1) * per].contiguous()   # the rank's own pool
        d = sdv.hnd_head_slice_descriptors(
            token_groups=groups, src_heads=per, src_head_begin=0, dst_heads=H,
            dst_head_begin=rank * per, num_heads=per, head_dim=w.head_dim, kv_dtype=pool.dtype,
            src_page_offsets=np.array(pages) * send_page_b,
            dst_page_offsets=np.array(pages) * recv_page_b)
        sdv.copy_descriptors(sender, recv, torch.from_numpy(d).to(DEV), dev_err=dev_err)
    torch.cuda.synchronize()
    return pool, recv, pages


def test_grouped_transfer_is_bitwise_exact():
    c = W.make_dense_case(CASE)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    pool, recv, pages = _transfer(c, 4, err)
    assert int(err.item()) == 0
    assert _logical_digests(recv, pages) == _logical_digests(pool, pages)
    idx = torch.tensor(pages, device=DEV)
    assert torch.equal(recv[idx].view(torch.int16), pool[idx].view(torch.int16))


def test_contiguous_slice_mapping_is_wrong_after_group0():
    c = W.make_dense_case(CASE)
    pool, recv, pages = _transfer(c, 1)
    got, ref = _logical_digests(recv, pages), _logical_digests(pool, pages)
    assert all(got[k] != ref[k] for k in ref)
    idx = torch.tensor(pages, device=DEV)
    # rank 0's heads in group 0 land where they belong
    assert torch.equal(recv[idx][:, 0, 0:2].view(torch.int16), pool[idx][:, 0, 0:2].view(torch.int16))
    assert not torch.equal(recv[idx][:, 1:, 0:2].view(torch.int16), pool[idx][:, 1:, 0:2].view(torch.int16))


def test_attention_over_the_received_pool():
    c = W.make_dense_case(CASE)
    _, recv, _ = _transfer(c, 4)
    run = DenseRun(c)
    run.pool = recv
    view, offs = run.view()
    out = run.attend(view, offs, num_splits=2)
    torch.cuda.synchronize()
    ok, worst = tol_ok(out_numpy(out[:run.n]), dense_oracle(c), "bf16")
    assert ok, worst


def test_copy_range_is_flagged_and_skipped():
    src = torch.arange(4096, dtype=torch.int32, device=DEV)
    dst = torch.zeros(4096, dtype=torch.int32, device=DEV)
    descs = torch.tensor([[0, 0, 1024],              # fine
                          [0, 16380, 64],            # past the end of dst
                          [8, 2048, 16],             # off the 16-byte grid
                          [1024, 4096, 1024]], dtype=torch.int64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    sdv.copy_descriptors(src, dst, descs, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & sdv._lib.DEVERR_COPY_RANGE
    d = dst.cpu().numpy()
    assert np.array_equal(d[:256], np.arange(256))
    assert np.array_equal(d[1024:1280], np.arange(256, 512))
    assert not d[256:1024].any() and not d[1280:].any()
