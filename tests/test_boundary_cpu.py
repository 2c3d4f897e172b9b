"""The C-ABI library on a machine without a GPU: it loads, exports every entry point
include/sdv.h declares, and rejects bad arguments on the host before any HIP call
(so no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

from speculative_decode_verify_p128_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = C.c_void_p(0x10000)          # never dereferenced: every call below fails validation


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sdv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\(", text, flags=re.M)))


def test_header_declarations_are_all_exported():
    names = _declared_functions()
    assert {"kv_subpage_view_init", "proxy_page_scores", "ladder_topk_pages",
            "verify_attention_dense", "verify_attention_sparse", "lse_combine"} <= set(names)
    lib = C.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(L.SIGNATURES) >= set(names)


def _geom(**kw):
    g = dict(phys_page=128, sub_page=32, num_kv_heads=4, head_dim=128, slot_stride=8,
             kv_offset=1, num_layers=1, num_slots=100, pool_index_scale=8, kv_dtype=L.SDV_BF16,
             k_scale=1.0, v_scale=1.0, k_root=0x10000)
    g.update(kw)
    return L.SubpageGeom(**g)


def _view_init(geom, B=1, max_blocks=4):
    lib = L.load()
    view = L.SubpageView()
    st = lib.kv_subpage_view_init(C.byref(geom), FAKE, B, max_blocks, max_blocks, FAKE,
                                  C.byref(view), None, None)
    return st, lib.sdv_last_error().decode(), view


@pytest.mark.parametrize("field,value", [("phys_page", 64), ("sub_page", 16), ("kv_offset", 2),
                                         ("kv_offset", 0), ("num_layers", 2), ("slot_stride", 1),
                                         ("head_dim", 96), ("num_kv_heads", 0),
                                         ("num_slots", 0), ("num_slots", 1 << 28)])
def test_view_geometry_rejections(field, value):
    st, msg, _ = _view_init(_geom(**{field: value}))
    assert st == L.SDV_ERR_GEOMETRY
    assert msg.startswith("native P128 draft view unavailable")


def test_view_accepts_pool_scale_different_from_stride():
    # The pages' hybrid pool: index scale 171 against a draft slot stride of 8.  With
    # B = 0 nothing is launched, so the geometry check alone decides.
    st, msg, view = _view_init(_geom(pool_index_scale=171, slot_stride=8), B=0)
    assert st == L.SDV_OK, msg
    assert view.index_scale == 8 and view.num_sub_pages == 4 * (99 * 8 + 2)


def test_view_other_rejections():
    assert _view_init(_geom(kv_dtype=7))[0] == L.SDV_ERR_DTYPE
    assert _view_init(_geom(k_root=0))[0] == L.SDV_ERR_NULL_POINTER
    assert _view_init(_geom(k_root=0x10008))[0] == L.SDV_ERR_GEOMETRY
    assert _view_init(_geom(k_scale=0.0))[0] == L.SDV_ERR_SHAPE
    lib = L.load()
    view = L.SubpageView()
    assert lib.kv_subpage_view_init(C.byref(_geom()), FAKE, 1, 4, 3, FAKE, C.byref(view), None,
                                    None) == L.SDV_ERR_SHAPE
    assert lib.kv_subpage_view_init(None, FAKE, 1, 4, 4, FAKE, C.byref(view), None,
                                    None) == L.SDV_ERR_NULL_POINTER


def _good_view():
    st, msg, view = _view_init(_geom(), B=0)
    assert st == 0, msg
    return view


def _dense(view, **kw):
    a = dict(q=FAKE, q_dt=L.SDV_BF16, qo=FAKE, kv=FAKE, B=2, max_qo=4, Hq=64, offs=FAKE,
             msp=64, scale=0.088, splits=1, ws=None, ws_bytes=0, out=FAKE, out_dt=L.SDV_BF16)
    a.update(kw)
    return L.load().verify_attention_dense(
        a["q"], a["q_dt"], a["qo"], a["kv"], a["B"], a["max_qo"], a["Hq"], C.byref(view),
        a["offs"], a["msp"], a["scale"], a["splits"], a["ws"], a["ws_bytes"], a["out"],
        a["out_dt"], None, None)


def test_dense_rejections():
    v = _good_view()
    assert _dense(v, q_dt=L.SDV_F32) == L.SDV_ERR_DTYPE          # f32 q with bf16 kv
    assert _dense(v, out_dt=L.SDV_FP8_E4M3) == L.SDV_ERR_DTYPE
    assert _dense(v, Hq=66) == L.SDV_ERR_SHAPE                    # not a multiple of Hkv
    assert _dense(v, max_qo=5) == L.SDV_ERR_SHAPE                 # 16 x 5 rows > 64
    assert _dense(v, max_qo=0) == L.SDV_ERR_SHAPE
    assert _dense(v, msp=0) == L.SDV_ERR_SHAPE
    assert _dense(v, scale=float("nan")) == L.SDV_ERR_SHAPE
    assert _dense(v, splits=0) == L.SDV_ERR_SHAPE
    assert _dense(v, q=None) == L.SDV_ERR_NULL_POINTER
    assert _dense(v, splits=4) == L.SDV_ERR_WORKSPACE             # no workspace given
    need = L.load().sdv_workspace_bytes(L.SDV_OP_VERIFY_DENSE, 8, 64, 128, 4)
    assert need >= 4 * 8 * 64 * 129 * 4
    assert _dense(v, splits=4, ws=FAKE, ws_bytes=need - 1) == L.SDV_ERR_WORKSPACE
    assert _dense(v, q=C.c_void_p(0x10008)) == L.SDV_ERR_SHAPE    # q not 16-byte aligned
    assert _dense(v, out=C.c_void_p(0x10004)) == L.SDV_ERR_SHAPE  # out not 16-byte aligned
    assert _dense(v, B=0) == L.SDV_OK                             # nothing to do
    assert _dense(v, offs=None) == L.SDV_ERR_NULL_POINTER
    # a split holds at most 1024 sub-pages: 2048 need two splits
    assert _dense(v, msp=2048) == L.SDV_ERR_SHAPE
    assert _dense(v, msp=2048, splits=2) == L.SDV_ERR_WORKSPACE   # accepted, needs a workspace
    empty = L.SubpageView()
    assert _dense(empty) != L.SDV_OK


def _dense_view(view, **kw):
    a = dict(q=FAKE, q_dt=L.SDV_BF16, qo=FAKE, kv=FAKE, B=2, max_qo=4, Hq=64, bt=FAKE, mb=16,
             bts=16, scale=0.088, splits=1, ws=None, ws_bytes=0, out=FAKE, out_dt=L.SDV_BF16)
    a.update(kw)
    return L.load().verify_attention_dense_view(
        a["q"], a["q_dt"], a["qo"], a["kv"], a["B"], a["max_qo"], a["Hq"], C.byref(view),
        a["bt"], a["mb"], a["bts"], a["scale"], a["splits"], a["ws"], a["ws_bytes"], a["out"],
        a["out_dt"], None, None)


def test_dense_view_rejections():
    v = _good_view()
    assert _dense_view(v, mb=0) == L.SDV_ERR_SHAPE
    assert _dense_view(v, bts=8) == L.SDV_ERR_SHAPE               # row stride below width
    assert _dense_view(v, mb=1 << 25, bts=1 << 25) == L.SDV_ERR_SHAPE
    assert _dense_view(v, bt=None) == L.SDV_ERR_NULL_POINTER
    assert _dense_view(v, q_dt=L.SDV_F32) == L.SDV_ERR_DTYPE
    assert _dense_view(v, max_qo=5) == L.SDV_ERR_SHAPE
    assert _dense_view(v, splits=4) == L.SDV_ERR_WORKSPACE
    assert _dense_view(v, out=None) == L.SDV_ERR_NULL_POINTER
    assert _dense_view(v, B=0) == L.SDV_OK
    assert _dense_view(L.SubpageView()) != L.SDV_OK


def _kv(**kw):
    d = dict(k=0x10000, v=0x20000, page_stride=4 * 128 * 128, num_pages=10, page_size=128,
             num_kv_heads=4, head_dim=128, kv_dtype=L.SDV_BF16, k_scale=1.0, v_scale=1.0)
    d.update(kw)
    return L.PagedKV(**d)


def _proxy(kv, **kw):
    a = dict(q_dt=L.SDV_BF16, B=2, max_qo=4, Hq=16, max_pages=8, bt_stride=8, scores=FAKE)
    a.update(kw)
    return L.load().proxy_page_scores(FAKE, a["q_dt"], FAKE, FAKE, a["B"], a["max_qo"], a["Hq"],
                                      C.byref(kv), FAKE, a["max_pages"], a["bt_stride"],
                                      a["scores"], None, None)


def test_proxy_rejections():
    assert _proxy(_kv(page_size=64)) == L.SDV_ERR_GEOMETRY
    assert _proxy(_kv(head_dim=80)) == L.SDV_ERR_SHAPE
    assert _proxy(_kv(page_stride=100)) == L.SDV_ERR_SHAPE
    assert _proxy(_kv(k=0)) == L.SDV_ERR_NULL_POINTER
    assert _proxy(_kv(k=0x10004)) == L.SDV_ERR_SHAPE                # misaligned pool
    assert _proxy(_kv(kv_dtype=9)) == L.SDV_ERR_DTYPE
    assert _proxy(_kv(), q_dt=L.SDV_FP8_E4M3) == L.SDV_ERR_DTYPE
    assert _proxy(_kv(), bt_stride=4) == L.SDV_ERR_SHAPE
    assert _proxy(_kv(), max_qo=64) == L.SDV_ERR_SHAPE              # q staging too large
    assert _proxy(_kv(), scores=None) == L.SDV_ERR_NULL_POINTER
    assert _proxy(_kv(), B=65536) == L.SDV_ERR_SHAPE                # launch grid limits
    assert _proxy(_kv(), max_pages=2 * 65535 + 1, bt_stride=2 * 65535 + 1) == L.SDV_ERR_SHAPE
    assert _proxy(_kv(), B=0) == L.SDV_OK


def _topk(**kw):
    a = dict(B=2, max_qo=4, Hkv=4, max_pages=8, page=128, k=2, idx=FAKE)
    a.update(kw)
    return L.load().ladder_topk_pages(FAKE, FAKE, FAKE, a["B"], a["max_qo"], a["Hkv"],
                                      a["max_pages"], a["page"], a["k"], a["idx"], None, None, None)


def test_topk_rejections():
    assert _topk(page=32) == L.SDV_ERR_GEOMETRY
    assert _topk(k=0) == L.SDV_ERR_SHAPE
    assert _topk(max_pages=5000) == L.SDV_ERR_SHAPE
    assert _topk(B=65536) == L.SDV_ERR_SHAPE                        # launch grid limit
    assert _topk(idx=None) == L.SDV_ERR_NULL_POINTER
    assert _topk(B=0) == L.SDV_OK


def _sparse(kv, **kw):
    a = dict(q=FAKE, q_dt=L.SDV_BF16, B=2, max_qo=4, Hq=16, max_pages=8, bt=8, k=2, splits=1,
             out=FAKE, out_dt=L.SDV_BF16)
    a.update(kw)
    return L.load().verify_attention_sparse(
        a["q"], a["q_dt"], FAKE, FAKE, a["B"], a["max_qo"], a["Hq"], C.byref(kv), FAKE,
        a["max_pages"], a["bt"], FAKE, a["k"], 0.088, a["splits"], None, 0, a["out"], a["out_dt"],
        None, None)


def test_sparse_rejections():
    assert _sparse(_kv(), q_dt=L.SDV_F32) == L.SDV_ERR_DTYPE
    assert _sparse(_kv(kv_dtype=L.SDV_F32), q_dt=L.SDV_BF16) == L.SDV_ERR_DTYPE
    assert _sparse(_kv(), k=0) == L.SDV_ERR_SHAPE
    assert _sparse(_kv(), k=200) == L.SDV_ERR_SHAPE                # 4 x 200 > 512
    assert _sparse(_kv(), max_pages=20000, bt=20000) == L.SDV_ERR_SHAPE
    assert _sparse(_kv(), splits=2) == L.SDV_ERR_WORKSPACE
    assert _sparse(_kv(), Hq=15) == L.SDV_ERR_SHAPE
    assert _sparse(_kv(), q=C.c_void_p(0x10002)) == L.SDV_ERR_SHAPE   # q not 16-byte aligned
    assert _sparse(_kv(), out=C.c_void_p(0x10008)) == L.SDV_ERR_SHAPE # out not 16-byte aligned
    assert _sparse(_kv(), B=0) == L.SDV_OK


def _select(kv, **kw):
    a = dict(q=FAKE, q_dt=L.SDV_BF16, B=2, max_qo=4, Hq=16, max_pages=8, bt=8, scores=FAKE, k=2,
             idx=FAKE, splits=1, out=FAKE, out_dt=L.SDV_BF16)
    a.update(kw)
    return L.load().verify_attention_sparse_select(
        a["q"], a["q_dt"], FAKE, FAKE, a["B"], a["max_qo"], a["Hq"], C.byref(kv), FAKE,
        a["max_pages"], a["bt"], a["scores"], a["k"], a["idx"], None, 0.088, a["splits"], None, 0,
        a["out"], a["out_dt"], None, None)


def test_select_rejections():
    # (every case fails on the host before a launch)
    assert _select(_kv(), scores=None) == L.SDV_ERR_NULL_POINTER
    assert _select(_kv(), q_dt=L.SDV_F32) == L.SDV_ERR_DTYPE
    assert _select(_kv(), k=200) == L.SDV_ERR_SHAPE                # 4 x 200 > 512
    # over 1024 pages the selection runs in a launch of its own into topk_idx ...
    assert _select(_kv(), max_pages=2000, bt=2000, idx=None) == L.SDV_ERR_NULL_POINTER
    # ... which takes up to 4096 pages
    assert _select(_kv(), max_pages=5000, bt=5000) == L.SDV_ERR_SHAPE
    assert _select(_kv(), splits=2) == L.SDV_ERR_WORKSPACE
    assert _select(_kv(), B=0) == L.SDV_OK


def _paged(kv, **kw):
    a = dict(q=FAKE, q_dt=L.SDV_BF16, B=2, max_qo=4, Hq=16, max_pages=8, bt=8, splits=1,
             out=FAKE, out_dt=L.SDV_BF16)
    a.update(kw)
    return L.load().verify_attention_paged(
        a["q"], a["q_dt"], FAKE, FAKE, a["B"], a["max_qo"], a["Hq"], C.byref(kv), FAKE,
        a["max_pages"], a["bt"], 0.088, a["splits"], None, 0, a["out"], a["out_dt"], None, None)


def test_paged_rejections():
    assert _paged(_kv(), q_dt=L.SDV_F32) == L.SDV_ERR_DTYPE           # matrix-core kernels only
    assert _paged(_kv(kv_dtype=L.SDV_F32)) == L.SDV_ERR_DTYPE
    assert _paged(_kv(), Hq=64, max_qo=5) == L.SDV_ERR_SHAPE          # 16 x 5 > 64 rows
    assert _paged(_kv(), max_pages=300, bt=300) == L.SDV_ERR_SHAPE     # 1200 blocks in one split
    assert _paged(_kv(), splits=2, max_pages=300, bt=300) == L.SDV_ERR_WORKSPACE
    assert _paged(_kv(), bt=4) == L.SDV_ERR_SHAPE                     # stride < max_pages
    assert _paged(_kv(), q=C.c_void_p(0x10004)) == L.SDV_ERR_SHAPE
    assert _paged(_kv(), out=None) == L.SDV_ERR_NULL_POINTER
    assert _paged(_kv(), B=0) == L.SDV_OK


def test_greedy_accept_workspace_bytes():
    lib = L.load()
    ws = lib.sdv_greedy_accept_workspace_bytes
    # one part per 1024 16-byte vectors: 8192 bf16 or 4096 f32 logits; 8 bytes per (row, part)
    assert ws(64, 4, 131072, L.SDV_BF16) == 64 * 4 * 16 * 8
    assert ws(64, 4, 131072, L.SDV_F32) == 64 * 4 * 32 * 8
    assert ws(3, 2, 8200, L.SDV_BF16) == 3 * 2 * 2 * 8
    assert ws(3, 2, 8, L.SDV_BF16) == 3 * 2 * 1 * 8
    assert ws(0, 4, 1024, L.SDV_BF16) == 0
    assert ws(2, 4, 1024, L.SDV_FP8_E4M3) == 0


def test_greedy_accept_rejections():
    lib = L.load()
    big = 1 << 20
    args = lambda dt, vocab, logits=FAKE, tokens=FAKE, ws=FAKE, wsb=big: (  # noqa: E731
        logits, dt, vocab, tokens, FAKE, FAKE, 2, 4, ws, wsb, FAKE, FAKE, FAKE, FAKE, None, None)
    assert lib.greedy_accept(*args(L.SDV_FP8_E4M3, 1024)) == L.SDV_ERR_DTYPE
    assert lib.greedy_accept(*args(L.SDV_BF16, 1020)) == L.SDV_ERR_SHAPE     # not a multiple of 8
    assert lib.greedy_accept(*args(L.SDV_F32, 0)) == L.SDV_ERR_SHAPE
    assert lib.greedy_accept(*args(L.SDV_BF16, 1024, tokens=None)) == L.SDV_ERR_NULL_POINTER
    assert lib.greedy_accept(*args(L.SDV_BF16, 1024, ws=None)) == L.SDV_ERR_NULL_POINTER
    assert lib.greedy_accept(*args(L.SDV_BF16, 1024, logits=C.c_void_p(0x10008))) == L.SDV_ERR_SHAPE
    # 2 requests x 4 rows x 2 parts x 8 bytes = 128
    assert lib.greedy_accept(*args(L.SDV_BF16, 16384, wsb=127)) == L.SDV_ERR_WORKSPACE
    assert lib.greedy_accept(*args(L.SDV_BF16, 16384, ws=C.c_void_p(0x10004))) == L.SDV_ERR_SHAPE


def test_read_units_probe_rejections():
    lib = L.load()
    f = lib.sdv_read_units_probe
    assert f(FAKE, 1 << 20, FAKE, 0, 8192, FAKE, 64, None) == L.SDV_OK          # nothing to read
    assert f(None, 1 << 20, FAKE, 4, 8192, FAKE, 64, None) == L.SDV_ERR_NULL_POINTER
    assert f(FAKE, 1 << 20, FAKE, 4, 1000, FAKE, 64, None) == L.SDV_ERR_SHAPE
    assert f(FAKE, 1 << 20, FAKE, 4, 8192, FAKE, 0, None) == L.SDV_ERR_SHAPE
    assert f(C.c_void_p(0x10008), 1 << 20, FAKE, 4, 8192, FAKE, 64, None) == L.SDV_ERR_SHAPE


def test_combine_and_helpers():
    lib = L.load()
    assert lib.lse_combine(FAKE, FAKE, 0, 4, 4, 128, FAKE, 0, None, None) == L.SDV_ERR_SHAPE
    assert lib.lse_combine(FAKE, FAKE, 2, 4, 4, 100, FAKE, 0, None, None) == L.SDV_ERR_SHAPE
    assert lib.lse_combine(FAKE, FAKE, 2, 4, 4, 128, FAKE, 2, None, None) == L.SDV_ERR_DTYPE
    assert lib.lse_combine(None, FAKE, 2, 4, 4, 128, FAKE, 0, None, None) == L.SDV_ERR_NULL_POINTER
    assert lib.lse_combine(FAKE, FAKE, 2, 0, 4, 128, FAKE, 0, None, None) == L.SDV_OK
    assert lib.sdv_status_string(3).decode().startswith("unsupported geometry")
    assert lib.sdv_fill_u32(FAKE, 17, 0, None) == L.SDV_ERR_SHAPE


def test_workspace_bytes_per_op():
    lib = L.load()
    f = lib.sdv_workspace_bytes
    units = 4 * 8 * 64                              # splits x rows x heads
    pad = lambda x: (x + 255) // 256 * 256          # noqa: E731
    for op in (L.SDV_OP_VERIFY_DENSE, L.SDV_OP_VERIFY_SPARSE, L.SDV_OP_VERIFY_PAGED):
        assert f(op, 8, 64, 128, 4) == pad(units * 128 * 4) + pad(units * 4)
        assert f(op, 8, 64, 128, 1) == 0            # one split: no partials
        assert f(op, 0, 64, 128, 4) == 0
    assert f(0, 8, 64, 128, 4) == 0                 # not an attention op
    assert f(99, 8, 64, 128, 4) == 0


def test_product_library_holds_no_kernel_selection_state():
    """The product library exports no setter that changes what later calls compute and no
    cross-check entry point; the cross-check build exports per-call family variants."""
    lib = C.CDLL(L.LIB_PATH)
    assert not hasattr(lib, "sdv_set_kernel_family")
    for name in L.XCHECK_SIGNATURES:
        assert not hasattr(lib, name), name
    x = L.load_xcheck()
    for name in L.XCHECK_SIGNATURES:
        assert hasattr(x, name), name
    assert not hasattr(x, "sdv_set_kernel_family")


def test_xcheck_rejects_unknown_family_before_any_launch():
    x = L.load_xcheck()
    v = _good_view()
    args = (FAKE, L.SDV_BF16, FAKE, FAKE, 2, 4, 64, C.byref(v), FAKE, 16, 16, 0.088, 1, None, 0,
            FAKE, L.SDV_BF16, None, None)
    for fam in (2, 7, -1):
        assert x.sdv_xcheck_verify_attention_dense_view(fam, *args) == L.SDV_ERR_SHAPE
        assert "kernel family" in x.sdv_last_error().decode()
    # a valid family still validates the arguments on the host (null q)
    bad = (None,) + args[1:]
    assert x.sdv_xcheck_verify_attention_dense_view(L.FAMILY_VALU, *bad) == L.SDV_ERR_NULL_POINTER


def test_dense_view_noalloc_host_checks():
    lib = L.load()
    v = _good_view()
    f = lambda B, splits, Hq=64: lib.verify_attention_dense_view_noalloc(  # noqa: E731
        FAKE, L.SDV_BF16, FAKE, FAKE, B, 4, Hq, C.byref(v), FAKE, 16, 16, 0.088, splits, FAKE,
        L.SDV_BF16, None, None)
    # partials of 4096 splits x 8 rows x 64 heads x 128 channels exceed the scratch: refused
    # before any HIP call
    assert f(2, 4096) == L.SDV_ERR_WORKSPACE
    assert "scratch" in lib.sdv_last_error().decode()
    assert f(0, 4) == L.SDV_OK                          # nothing to do
    assert f(2, 1, Hq=66) == L.SDV_ERR_SHAPE            # argument checks as the workspace entry
