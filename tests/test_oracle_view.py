"""Pins for the oracle's paged addressing (CPU only).

A pool whose every element holds its own flat index lets a gathered value name the
physical (page, group, head, token, channel) it came from; the expected coordinates
are written from the pages' own statements, via numpy.ravel_multi_index, not from
the oracle's P32 index arithmetic.
"""
import hashlib
import json
import os

import numpy as np

import oracle
from oracle.view import apply_descriptors

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _coded_pool(num_pages, H, d):
    shape = (num_pages, 4, H, 32, d)
    return np.arange(np.prod(shape), dtype=np.int64).reshape(shape), shape


def _check_view(stride, root, H, d, kv_len, seed):
    rng = np.random.default_rng(seed)
    num_slots = 12
    pool, shape = _coded_pool(num_slots * stride, H, d)
    n_blocks = -(-kv_len // 128)
    W = n_blocks + 2                                        # two padding entries
    bt = np.zeros((1, W), dtype=np.int64)
    bt[0, :n_blocks] = rng.permutation(np.arange(1, num_slots))[:n_blocks]
    offs = oracle.subpage_offsets(bt, stride)
    root_elem = root * 4 * H * 32 * d
    K, V = oracle.gather_subpage_view(pool.reshape(-1)[root_elem:], offs[0], kv_len, H, d)
    j = np.arange(kv_len)[:, None, None]
    h = np.arange(H)[None, :, None]
    c = np.arange(d)[None, None, :]
    slot = bt[0, j // 128]
    # [PR18066] view-scale commit: slot s's K page is s * stride from the draft layer's
    # K page, V is the next page.  [PR17835] item 2: the page is [4, head, 32, d].
    k_page = root + slot * stride
    exp_k = np.ravel_multi_index(np.broadcast_arrays(k_page, (j % 128) // 32, h, j % 32, c), shape)
    exp_v = np.ravel_multi_index(np.broadcast_arrays(k_page + 1, (j % 128) // 32, h, j % 32, c), shape)
    assert np.array_equal(K, exp_k)
    assert np.array_equal(V, exp_v)
    return offs


def test_view_gather_names_the_right_physical_elements():
    for stride, root, H, d, kv in ((2, 0, 2, 64, 300), (8, 6, 4, 16, 517), (8, 6, 2, 8, 129),
                                   (3, 1, 1, 4, 31), (8, 0, 4, 8, 1)):
        _check_view(stride, root, H, d, kv, seed=stride * 100 + kv)


def test_view_padding_addresses_slot0():
    # [PR18066] dead-code commit: padded block-table entries stay 0 and address
    # valid slot-0 memory.
    bt = np.zeros((1, 3), dtype=np.int64)
    offs = oracle.subpage_offsets(bt, 8)
    assert list(offs[0, 0]) == [0, 1, 2, 3] * 3
    assert list(offs[0, 1]) == [4, 5, 6, 7] * 3


def test_view_geometry_golden():
    # The pages print a hybrid-pool geometry: pool index scale 171 with a draft slot
    # stride of 8.  The view's offsets depend on the stride only.
    with open(os.path.join(GOLDEN, "view_geometry.json")) as f:
        g = json.load(f)
    bt = np.array([g["slots"]], dtype=np.int64)
    offs = oracle.subpage_offsets(bt, g["draft_slot_stride"])
    for i, s in enumerate(g["slots"]):
        for grp in range(4):
            k32 = offs[0, 0, 4 * i + grp]
            v32 = offs[0, 1, 4 * i + grp]
            assert k32 // 4 == s * g["draft_slot_stride"]          # K at s * stride
            assert v32 // 4 == s * g["draft_slot_stride"] + 1      # V at s * stride + 1
            assert k32 % 4 == grp and v32 % 4 == grp


def test_hnd_gather_names_the_right_physical_elements():
    rng = np.random.default_rng(3)
    P, H, d = 9, 3, 8
    shape = (P, H, 128, d)
    pool = np.arange(np.prod(shape), dtype=np.int64).reshape(shape)
    bt = rng.permutation(P)[:4]
    kv = 389
    seq = oracle.gather_hnd(pool, bt, kv)
    j = np.arange(kv)[:, None, None]
    h = np.arange(H)[None, :, None]
    c = np.arange(d)[None, None, :]
    exp = np.ravel_multi_index(np.broadcast_arrays(bt[j // 128], h, j % 128, c), shape)
    assert np.array_equal(seq, exp)


def _grouped_page(logical):           # logical [H, 128, d] -> grouped [4, H, 32, d]
    H, _, d = logical.shape
    return logical.reshape(H, 4, 32, d).transpose(1, 0, 2, 3).copy()


def test_grouped_head_slice_transfer_exact_and_contiguous_mapper_wrong_after_group0():
    # [PR17835] item 2: TP2 context ranks hold 2 of the 4 KV heads each, attention-DP
    # generation holds all 4.  One descriptor per token group reproduces the grouped
    # page exactly (checked with SHA-256, as in the pages' transfer proof); one
    # contiguous head slice per page is right only in the first P32 group.
    rng = np.random.default_rng(7)
    H, d = 4, 16
    logical = rng.standard_normal((H, 128, d)).astype(np.float32)
    truth = _grouped_page(logical)
    fixed = np.zeros_like(truth).reshape(-1)
    old = np.zeros_like(truth).reshape(-1)
    for rank, (h0, h1) in enumerate(((0, 2), (2, 4))):
        src = _grouped_page(logical[h0:h1]).reshape(-1)          # the rank's own page
        apply_descriptors(fixed, src, oracle.head_slice_grouped(H, h0, h1, d))
        apply_descriptors(old, src, oracle.head_slice_contiguous(H, h0, h1, d))
    fixed = fixed.reshape(truth.shape)
    old = old.reshape(truth.shape)
    assert hashlib.sha256(fixed.tobytes()).hexdigest() == hashlib.sha256(truth.tobytes()).hexdigest()
    assert np.array_equal(fixed, truth)
    # Old mapper: rank 0's heads 0-1 land correctly in group 0 only.
    assert np.array_equal(old[0, 0:2], truth[0, 0:2])
    for g in (1, 2, 3):
        assert not np.array_equal(old[g], truth[g])
