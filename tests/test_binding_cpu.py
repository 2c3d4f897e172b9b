"""The PyTorch binding's argument checks, on the CPU: every shape, dtype or device that
does not match what the C entry point will address is rejected before the call, so no
mismatch can turn into an out-of-bounds access on the GPU.  The tensors here are host
tensors, so a call that passed every shape check stops at the device check."""
import pytest
import torch

import speculative_decode_verify_p128_amd as sdv

B, QO, HQ, HKV, D, PAGES, K = 3, 4, 16, 4, 128, 8, 4
ROWS = B * QO


def _lens():
    return torch.tensor([0, 4, 8, 12], dtype=torch.int32), torch.tensor([300, 400, 500],
                                                                           dtype=torch.int32)


def _kv(d=D):
    k = torch.zeros((20, HKV, 128, d), dtype=torch.bfloat16)
    return sdv.PagedKV(k, k.clone())


def _q(rows=ROWS, hq=HQ, d=D, dtype=torch.bfloat16):
    return torch.zeros((rows, hq, d), dtype=dtype)


def _bt(b=B, w=PAGES):
    return torch.zeros((b, w), dtype=torch.int32)


def _scores(rows=ROWS, hkv=HKV, pages=PAGES):
    return torch.zeros((rows, hkv, pages), dtype=torch.float32)


def _raises_shape(fn, match=None):
    with pytest.raises(ValueError, match=match):
        fn()


def test_query_checks():
    ind, kvl = _lens()
    call = lambda q: sdv.proxy_page_scores(q, ind, kvl, _kv(), _bt(), max_qo_len=QO)  # noqa: E731
    _raises_shape(lambda: call(_q(d=64)), "head_dim")              # d 64 over a d 128 pool
    _raises_shape(lambda: call(_q(hq=18)), "multiple")             # 18 heads over 4 KV heads
    _raises_shape(lambda: call(_q(rows=ROWS - 1)), "rows")          # below B * max_qo_len
    with pytest.raises(TypeError):
        call(_q(dtype=torch.float16))
    _raises_shape(lambda: call(_q()), "GPU")                       # right shapes, host memory


def test_lengths_and_table_checks():
    ind, kvl = _lens()
    _raises_shape(lambda: sdv.proxy_page_scores(_q(), ind[:3], kvl, _kv(), _bt(), max_qo_len=QO),
                  "B \\+ 1")
    _raises_shape(lambda: sdv.proxy_page_scores(_q(), ind, kvl, _kv(), _bt(b=2), max_qo_len=QO),
                  "block_table")
    with pytest.raises(TypeError):
        sdv.proxy_page_scores(_q(), ind, kvl, _kv(), _bt().long(), max_qo_len=QO)


def test_scores_checks():
    ind, kvl = _lens()
    f = lambda s: sdv.proxy_page_scores(_q(), ind, kvl, _kv(), _bt(), max_qo_len=QO,  # noqa: E731
                                        scores=s)
    _raises_shape(lambda: f(_scores(rows=ROWS - 1)), "scores")
    _raises_shape(lambda: f(_scores(hkv=2)), "scores")
    _raises_shape(lambda: f(_scores(pages=PAGES - 1)), "scores")
    g = lambda s, **kw: sdv.ladder_topk_pages(s, ind, kvl, max_qo_len=QO, top_k=K, **kw)  # noqa: E731
    _raises_shape(lambda: g(_scores(rows=ROWS - 1)), "scores")
    _raises_shape(lambda: g(_scores(), topk_idx=torch.zeros((ROWS, HKV, K - 1), dtype=torch.int32)),
                  "topk_idx")
    _raises_shape(lambda: g(_scores(), topk_cnt=torch.zeros((ROWS - 1, HKV), dtype=torch.int32)),
                  "topk_cnt")


def test_attention_output_checks():
    ind, kvl = _lens()
    idx = torch.zeros((ROWS, HKV, K), dtype=torch.int32)
    f = lambda **kw: sdv.verify_attention_sparse(_q(), ind, kvl, _kv(), _bt(), idx,  # noqa: E731
                                                 max_qo_len=QO, softmax_scale=0.088, **kw)
    _raises_shape(lambda: f(out=torch.zeros((ROWS - 1, HQ, D), dtype=torch.bfloat16)), "out")
    _raises_shape(lambda: f(out=torch.zeros((ROWS, HQ, 64), dtype=torch.bfloat16)), "out")
    with pytest.raises(TypeError):
        f(out=torch.zeros((ROWS, HQ, D), dtype=torch.float16))
    _raises_shape(lambda: sdv.verify_attention_sparse(
        _q(), ind, kvl, _kv(), _bt(), idx[:ROWS - 1], max_qo_len=QO, softmax_scale=0.088),
        "topk_idx")
    # paged and selection wrappers share the checks
    _raises_shape(lambda: sdv.verify_attention_paged(_q(d=64), ind, kvl, _kv(), _bt(),
                                                     max_qo_len=QO, softmax_scale=0.1), "head_dim")
    _raises_shape(lambda: sdv.verify_attention_sparse_select(
        _q(), ind, kvl, _kv(), _bt(), _scores(pages=PAGES + 1), max_qo_len=QO, top_k=K,
        softmax_scale=0.1), "scores")
    _raises_shape(lambda: sdv.verify_attention_sparse_select(
        _q(), ind, kvl, _kv(), _bt(), _scores(), max_qo_len=QO, top_k=K, softmax_scale=0.1,
        topk_cnt=torch.zeros((ROWS, HKV + 1), dtype=torch.int32)), "topk_cnt")
    _raises_shape(lambda: f(), "GPU")


def test_dense_checks():
    ind, kvl = _lens()
    view = sdv.SubpageView(sdv._lib.SubpageView(0, 1, HKV, D, 8, 10, 1.0, 1.0, 64),
                           torch.zeros(1, dtype=torch.bfloat16))
    offs = torch.zeros((B, 2, 64), dtype=torch.int32)
    _raises_shape(lambda: sdv.verify_attention_dense(_q(d=64), ind, kvl, view, offs, max_qo_len=QO,
                                                     softmax_scale=0.1), "head_dim")
    _raises_shape(lambda: sdv.verify_attention_dense(_q(), ind, kvl, view, offs[:2], max_qo_len=QO,
                                                     softmax_scale=0.1), "sub_offsets")
    _raises_shape(lambda: sdv.verify_attention_dense_view(_q(), ind, kvl, view, _bt(),
                                                          max_qo_len=QO, softmax_scale=0.1,
                                                          max_blocks=PAGES + 1), "max_blocks")
    _raises_shape(lambda: sdv.verify_attention_dense_view(_q(hq=6), ind, kvl, view, _bt(),
                                                          max_qo_len=QO, softmax_scale=0.1),
                  "multiple")


def test_staging_and_accept_checks():
    ind, kvl = _lens()
    kn = torch.zeros((ROWS, HKV, D), dtype=torch.bfloat16)
    _raises_shape(lambda: sdv.stage_verify_kv_paged(kn[:ROWS - 1], kn, ind, kvl, _kv(), _bt(),
                                                    max_qo_len=QO), "k_new")
    _raises_shape(lambda: sdv.stage_verify_kv_paged(kn, kn[..., :64], ind, kvl, _kv(), _bt(),
                                                    max_qo_len=QO), "v_new")
    logits = torch.zeros((ROWS, 1024), dtype=torch.bfloat16)
    tok = torch.zeros(ROWS, dtype=torch.int32)
    _raises_shape(lambda: sdv.greedy_accept(logits, tok[:5], ind, kvl, max_qo_len=QO), "tokens")
    outs = (torch.zeros(ROWS - 1, dtype=torch.int32), torch.zeros(B, dtype=torch.int32),
            torch.zeros((B, QO), dtype=torch.int32), torch.zeros(B, dtype=torch.int32))
    _raises_shape(lambda: sdv.greedy_accept(logits, tok, ind, kvl, max_qo_len=QO, outs=outs),
                  "targets")


def test_combine_checks():
    po = torch.zeros((2, 5, 3, 64), dtype=torch.float32)
    _raises_shape(lambda: sdv.lse_combine(po, torch.zeros((2, 5, 4))), "partial_lse")
    _raises_shape(lambda: sdv.lse_combine(po, torch.zeros((2, 5, 3)),
                                          out=torch.zeros((4, 3, 64))), "out")
    _raises_shape(lambda: sdv.lse_combine(po, torch.zeros((2, 5, 3))), "GPU")
