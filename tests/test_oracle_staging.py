"""Pins of the oracle's ladder KV slot staging.  Staged rows are read back through the
gathers (themselves pinned against coordinate-encoded pools): the new tokens appear at
logical positions kv_len - qo_len .. kv_len - 1, everything else is untouched, and a
later correction that shortens one request across a page boundary re-stages only that
request."""
import numpy as np

import oracle
from oracle.staging import stage_paged, stage_view

RNG = np.random.default_rng(7)


def _paged_setup(B=3, H=2, d=8, pages_per_req=3, spare=2):
    num_pages = B * pages_per_req + spare
    perm = RNG.permutation(num_pages)
    bt = perm[: B * pages_per_req].reshape(B, pages_per_req)
    kp = RNG.integers(0, 2 ** 16, size=(num_pages, H, 128, d), dtype=np.uint16)
    vp = RNG.integers(0, 2 ** 16, size=(num_pages, H, 128, d), dtype=np.uint16)
    return bt, kp, vp


def _rows(qo, H, d):
    ind = np.concatenate([[0], np.cumsum(qo)])
    k = RNG.integers(0, 2 ** 16, size=(ind[-1], H, d), dtype=np.uint16)
    v = RNG.integers(0, 2 ** 16, size=(ind[-1], H, d), dtype=np.uint16)
    return ind, k, v


def test_stage_paged_round_trip_and_nothing_else_changes():
    bt, kp, vp = _paged_setup()
    qo = np.array([4, 1, 3])
    kv = np.array([130, 128, 255])          # request 0 crosses into page 1; 2 ends at 255
    ind, kn, vn = _rows(qo, 2, 8)
    kp2, vp2 = stage_paged(kp, vp, kn, vn, ind, kv, bt)
    changed = 0
    for r in range(3):
        for old, new, rows in ((kp, kp2, kn), (vp, vp2, vn)):
            before = oracle.gather_hnd(old, bt[r], int(kv[r]))
            after = oracle.gather_hnd(new, bt[r], int(kv[r]))
            s = int(kv[r] - qo[r])
            assert np.array_equal(after[:s], before[:s])
            assert np.array_equal(after[s:], rows[ind[r]:ind[r + 1]])
            changed += int(np.sum(before[s:] != rows[ind[r]:ind[r + 1]]))
    diff = int(np.sum(kp != kp2) + np.sum(vp != vp2))
    assert diff == changed                  # every changed element is a staged one


def test_stage_paged_page_crossing_writes_both_pages():
    bt, kp, vp = _paged_setup(B=1)
    qo, kv = np.array([4]), np.array([130])  # positions 126, 127 | 128, 129
    ind, kn, vn = _rows(qo, 2, 8)
    kp2, _ = stage_paged(kp, vp, kn, vn, ind, kv, bt)
    assert np.array_equal(kp2[bt[0, 0], :, 126], kn[0]) and np.array_equal(kp2[bt[0, 0], :, 127], kn[1])
    assert np.array_equal(kp2[bt[0, 1], :, 0], kn[2]) and np.array_equal(kp2[bt[0, 1], :, 1], kn[3])


def test_stage_view_round_trip():
    H, d, stride, slots, root = 2, 8, 2, 5, 3
    page_elems = 4 * H * 32 * d
    pool = RNG.integers(0, 2 ** 16, size=(slots * stride + root + 2) * page_elems, dtype=np.uint16)
    bt = np.array([[1, 3], [4, 2]])
    qo = np.array([3, 4])
    kv = np.array([33, 200])                 # 31, 32 straddle a P32 boundary; 196..199
    ind, kn, vn = _rows(qo, H, d)
    out = stage_view(pool, root * page_elems, kn, vn, ind, kv, bt, stride, H, d)
    offs = oracle.subpage_offsets(bt, stride)
    for r in range(2):
        k0, v0 = oracle.gather_subpage_view(pool[root * page_elems:], offs[r], int(kv[r]), H, d)
        k1, v1 = oracle.gather_subpage_view(out[root * page_elems:], offs[r], int(kv[r]), H, d)
        s = int(kv[r] - qo[r])
        assert np.array_equal(k1[:s], k0[:s]) and np.array_equal(v1[:s], v0[:s])
        assert np.array_equal(k1[s:], kn[ind[r]:ind[r + 1]])
        assert np.array_equal(v1[s:], vn[ind[r]:ind[r + 1]])
    assert np.array_equal(out[:root * page_elems], pool[:root * page_elems])


def _flat_table(bt, kv):
    """A flat page list laid out by each request's page count: the layout the pages
    describe being rebuilt from lengths.  Row r's pages start at the sum of the earlier
    rows' counts."""
    n = [-(-int(k) // 128) for k in kv]
    return np.concatenate([bt[r, :n[r]] for r in range(len(kv))]), np.concatenate([[0], np.cumsum(n)])


def test_overlap_correction_restages_only_the_corrected_request():
    bt, kp, vp = _paged_setup(B=3, pages_per_req=3)
    # step A: every request appends 4 tokens
    qo = np.array([4, 4, 4])
    kv_a = np.array([200, 131, 300])
    ind, kn_a, vn_a = _rows(qo, 2, 8)
    kp_a, vp_a = stage_paged(kp, vp, kn_a, vn_a, ind, kv_a, bt)
    # correction: request 1 keeps only 1 of its 4 tokens -> 128 positions, one page fewer
    kv_corr = np.array([200, 128, 300])
    # step B: the next 4 tokens of every request, at the corrected positions
    kv_b = kv_corr + 4
    _, kn_b, vn_b = _rows(qo, 2, 8)
    kp_b, _ = stage_paged(kp_a, vp_a, kn_b, vn_b, ind, kv_b, bt)
    for r in range(3):
        seq = oracle.gather_hnd(kp_b, bt[r], int(kv_b[r]))
        s = int(kv_b[r] - 4)
        assert np.array_equal(seq[s:], kn_b[ind[r]:ind[r + 1]])
        prev = oracle.gather_hnd(kp_a, bt[r], s)
        assert np.array_equal(seq[:s], prev)          # earlier tokens untouched
    # negative control: a flat page list rebuilt with the stale (pre-correction) counts
    # misbases the later request once request 1 drops a page
    flat_stale, start_stale = _flat_table(bt, kv_a)
    flat_new, start_new = _flat_table(bt, kv_corr)
    assert start_stale[2] != start_new[2]
    assert flat_stale[start_stale[2]] != flat_new[start_stale[2]]
