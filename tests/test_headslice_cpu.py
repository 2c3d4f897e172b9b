"""Grouped head-major head-slice transfer (CPU): the oracle's descriptor list is pinned
to the per-page slices of the pages' statement and to a byte-level reconstruction
checked with SHA-256; the library's host-side mapper (no GPU involved) must return the
same descriptors, integer for integer."""
import hashlib

import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_p128_amd as sdv
import speculative_decode_verify_p128_amd._lib as L

RNG = np.random.default_rng(11)


def test_descriptors_match_the_per_page_slices():
    H, d, e = 4, 16, 2
    for h0, h1 in ((0, 2), (2, 4), (1, 4)):
        grouped = oracle.head_slice_descriptors(4, h1 - h0, 0, H, h0, h1 - h0, d, e, [0], [0])
        assert [(dst, n) for _, dst, n in grouped] == \
            [(off * e, ln * e) for off, ln in oracle.head_slice_grouped(H, h0, h1, d)]
        flat = oracle.head_slice_descriptors(1, h1 - h0, 0, H, h0, h1 - h0, d, e, [0], [0])
        assert [(dst, n) for _, dst, n in flat] == \
            [(off * e, ln * e) for off, ln in oracle.head_slice_contiguous(H, h0, h1, d)]


def _grouped_bytes(logical):             # [H, 128, d] float32 -> grouped page bytes
    H, _, d = logical.shape
    return logical.reshape(H, 4, 32, d).transpose(1, 0, 2, 3).copy().view(np.uint8).reshape(-1)


def test_byte_copies_rebuild_every_head_exactly():
    """Two TP2 ranks (heads 0-1, 2-3) send grouped pages to a 4-head receiver: with one
    descriptor per token group every logical head is bitwise equal (SHA-256); with one
    contiguous slice per page only the first 32-token group survives."""
    H, d, P = 4, 16, 3
    logical = RNG.standard_normal((P, H, 128, d)).astype(np.float32)
    page_b = H * 128 * d * 4
    for groups, expect_exact in ((4, True), (1, False)):
        dst = np.zeros(P * page_b, dtype=np.uint8)
        for h0 in (0, 2):
            src = np.concatenate([_grouped_bytes(logical[p, h0:h0 + 2]) for p in range(P)])
            src_pages = np.arange(P) * (page_b // 2)
            dst_pages = np.arange(P) * page_b
            for so, do, n in oracle.head_slice_descriptors(groups, 2, 0, H, h0, 2, d, 4,
                                                           src_pages, dst_pages):
                dst[do:do + n] = src[so:so + n]
        got = dst.view(np.float32).reshape(P, 4, H, 32, d).transpose(0, 2, 1, 3, 4).reshape(P, H, 128, d)
        for h in range(H):
            same = hashlib.sha256(got[:, h].tobytes()).digest() == \
                hashlib.sha256(logical[:, h].tobytes()).digest()
            assert same == expect_exact
        if not expect_exact:
            assert np.array_equal(got[:, 0:2, :32], logical[:, 0:2, :32])   # group 0 of rank 0


@pytest.mark.parametrize("groups", [1, 2, 4])
@pytest.mark.parametrize("dt,eb", [(torch.bfloat16, 2), (torch.float8_e4m3fn, 1), (torch.float32, 4)])
def test_library_mapper_equals_oracle(groups, dt, eb):
    src_pages = RNG.integers(0, 1000, size=7) * 65536
    dst_pages = RNG.integers(0, 1000, size=7) * 131072
    got = sdv.hnd_head_slice_descriptors(token_groups=groups, src_heads=2, src_head_begin=0,
                                         dst_heads=4, dst_head_begin=2, num_heads=2, head_dim=128,
                                         kv_dtype=dt, src_page_offsets=src_pages,
                                         dst_page_offsets=dst_pages)
    ref = oracle.head_slice_descriptors(groups, 2, 0, 4, 2, 2, 128, eb, src_pages, dst_pages)
    assert got.tolist() == [list(x) for x in ref]


def test_library_mapper_rejections():
    kw = dict(token_groups=4, src_heads=2, src_head_begin=0, dst_heads=4, dst_head_begin=2,
              num_heads=2, head_dim=128, kv_dtype=torch.bfloat16, src_page_offsets=[0],
              dst_page_offsets=[0])
    for bad in (dict(token_groups=3), dict(dst_head_begin=3), dict(src_head_begin=1),
                dict(page_tokens=130)):
        with pytest.raises(L.SdvError):
            sdv.hnd_head_slice_descriptors(**{**kw, **bad})
    assert sdv.hnd_head_slice_descriptors(**{**kw, "src_page_offsets": [],
                                             "dst_page_offsets": []}).shape == (0, 3)
