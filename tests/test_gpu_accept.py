"""GPU parity of greedy acceptance against the oracle, bit for bit (integer outputs):
bf16 and f32 logits, rows with two equal maxima and with NaN, ragged qo_len including
decode rows, vocabularies that span several row parts (ragged last part, equal maxima in
different parts, NaN-only parts), the full benchmark vocabulary on sampled requests, a
reused workspace, repeated calls, and the length flag (the flagged request's rows still
get their targets)."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_p128_amd as sdv
import workloads as W

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from _parity import DEV

VOCAB_FULL = 131072


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


def _run(c, max_qo, err=None):
    return sdv.greedy_accept(c.logits.to(DEV), c.tokens.to(DEV), c.qo_indptr.to(DEV),
                             c.kv_len.to(DEV), max_qo_len=max_qo, dev_err=err)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("w", [W.SPARSE_BF16, W.RAGGED_MIXED], ids=lambda w: w.name)
def test_accept_bit_exact(w, dt):
    c = W.make_accept_case(w, 1024, dtype=dt, tie_rows=0.2, nan_rows=0.1)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    targets, accept, emitted, new_kv = _run(c, w.max_qo(), err)
    torch.cuda.synchronize()
    ref = oracle.greedy_accept_case(c.logits.float().numpy(), c.tokens.numpy(),
                                    c.qo_indptr.numpy(), c.lengths.kv)
    n = c.lengths.total_q
    assert int(err.item()) == 0
    assert np.array_equal(targets[:n].cpu().numpy(), ref["targets"])
    assert np.array_equal(accept.cpu().numpy(), ref["accept"])
    em = emitted.cpu().numpy()
    assert np.array_equal(em[:, :ref["emitted"].shape[1]], ref["emitted"])
    assert np.all(em[:, ref["emitted"].shape[1]:] == -1)
    assert np.array_equal(new_kv.cpu().numpy(), ref["new_kv"])


def _check(c, out):
    targets, accept, emitted, new_kv = out
    ref = oracle.greedy_accept_case(c.logits.float().numpy(), c.tokens.numpy(),
                                    c.qo_indptr.numpy(), c.lengths.kv)
    n = c.lengths.total_q
    assert np.array_equal(targets[:n].cpu().numpy(), ref["targets"])
    assert np.array_equal(accept.cpu().numpy(), ref["accept"])
    em = emitted.cpu().numpy()
    assert np.array_equal(em[:, :ref["emitted"].shape[1]], ref["emitted"])
    assert np.all(em[:, ref["emitted"].shape[1]:] == -1)
    assert np.array_equal(new_kv.cpu().numpy(), ref["new_kv"])
    return ref


@pytest.mark.parametrize("dt,vocab", [(torch.bfloat16, 3 * 8192 + 8), (torch.float32, 2 * 4096 + 4),
                                      (torch.bfloat16, 8192), (torch.float32, 3 * 4096 - 4)],
                         ids=["bf16_ragged_part", "f32_ragged_part", "bf16_one_part", "f32_3parts"])
def test_accept_several_parts(dt, vocab):
    w = W.RAGGED_MIXED.scaled(name="accept_parts", batch=24)
    c = W.make_accept_case(w, vocab, dtype=dt, tie_rows=0.3, nan_rows=0.2)
    x = c.logits
    per_part = 8192 if dt == torch.bfloat16 else 4096
    parts = -(-vocab // per_part)
    # hand-made rows: equal maxima in the last and the first part (the first wins), in two
    # later parts, an all-NaN row, an all -inf row, NaN everywhere but the last part, a
    # maximum in the one-vector tail
    big = 50.0
    x[0, :] = 0.0
    x[0, vocab - 3] = big
    x[0, 5] = big
    if parts > 2:
        x[1, :] = -1.0
        x[1, 2 * per_part + 1] = big
        x[1, per_part + 7] = big
    x[2, :] = float("nan")
    x[3, :] = float("-inf")
    x[4, :] = float("nan")
    x[4, (parts - 1) * per_part:] = -2.0
    x[4, vocab - 1] = -1.5
    x[5, :] = -3.0
    x[5, vocab - 1] = 4.0
    out = _run(c, w.max_qo())
    torch.cuda.synchronize()
    ref = _check(c, out)
    assert ref["targets"][0] == 5 and ref["targets"][2] == -1 and ref["targets"][3] == 0
    assert ref["targets"][4] == vocab - 1 and ref["targets"][5] == vocab - 1
    if parts > 2:
        assert ref["targets"][1] == per_part + 7


@pytest.mark.parametrize("dt,vocab", [(torch.bfloat16, 65 * 8192 + 8), (torch.float32, 70 * 4096 + 4)],
                         ids=["bf16_66_parts", "f32_71_parts"])
def test_accept_more_than_64_parts(dt, vocab):
    """Rows of more than 64 parts, whose keys the acceptance wave merges row by row (lanes
    over parts) instead of spreading (row, part) pairs over its lanes."""
    w = W.SPARSE_BF16.scaled(name="accept_wide", batch=2)
    c = W.make_accept_case(w, vocab, dtype=dt, tie_rows=0.4, nan_rows=0.2)
    x = c.logits
    per_part = 8192 if dt == torch.bfloat16 else 4096
    x[0, :] = -1.0
    x[0, 64 * per_part + 3] = 7.0                      # maximum in a part past the 64th
    x[0, 2] = 7.0                                      # ... and the same value in part 0: wins
    x[1, :] = -1.0
    x[1, vocab - 1] = 9.0                              # in the last, ragged part
    _check(c, _run(c, w.max_qo()))


def test_accept_reused_workspace_smaller_second_call():
    """One workspace and output set serve two calls in a row, the second with fewer
    requests and a smaller vocabulary: stale part results of the first call must not
    leak into the second."""
    w1 = W.RAGGED_MIXED.scaled(name="accept_ws1", batch=32)
    c1 = W.make_accept_case(w1, 4 * 8192, tie_rows=0.2, nan_rows=0.1)
    need = sdv.greedy_accept_workspace_bytes(w1.batch, w1.max_qo(), 4 * 8192, torch.bfloat16)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)
    out1 = sdv.greedy_accept(c1.logits.to(DEV), c1.tokens.to(DEV), c1.qo_indptr.to(DEV),
                             c1.kv_len.to(DEV), max_qo_len=w1.max_qo(), workspace=ws)
    torch.cuda.synchronize()
    _check(c1, out1)
    w2 = W.RAGGED_MIXED.scaled(name="accept_ws2", batch=5)
    c2 = W.make_accept_case(w2, 8192 + 64, tie_rows=0.2, nan_rows=0.1)
    out2 = sdv.greedy_accept(c2.logits.to(DEV), c2.tokens.to(DEV), c2.qo_indptr.to(DEV),
                             c2.kv_len.to(DEV), max_qo_len=w2.max_qo(), workspace=ws)
    torch.cuda.synchronize()
    _check(c2, out2)


def test_accept_repeated_calls_same_outputs():
    """Many calls on one workspace, with the host reading back in between: identical
    outputs every time."""
    w = W.SPARSE_BF16.scaled(name="accept_rep", batch=16)
    c = W.make_accept_case(w, 2 * 8192 + 16, tie_rows=0.3, nan_rows=0.1)
    dev_in = [t.to(DEV) for t in (c.logits, c.tokens, c.qo_indptr, c.kv_len)]
    need = sdv.greedy_accept_workspace_bytes(w.batch, w.max_qo(), 2 * 8192 + 16, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    first = None
    for _ in range(20):
        out = sdv.greedy_accept(*dev_in, max_qo_len=w.max_qo(), workspace=ws)
        got = [t.cpu().clone() for t in out]
        if first is None:
            first = got
            _check(c, out)
        else:
            for a, b in zip(first, got):
                assert torch.equal(a, b)


def test_accept_full_vocab_sampled():
    w = W.SPARSE_BF16
    c = W.make_accept_case(w, VOCAB_FULL, device=DEV)
    targets, accept, emitted, new_kv = _run(c, w.max_qo())
    torch.cuda.synchronize()
    logits = c.logits.float().cpu().numpy()
    tokens = c.tokens.cpu().numpy()
    ind = c.qo_indptr.cpu().numpy()
    for r in (0, 17, 40, w.batch - 1):
        a0, b0 = ind[r], ind[r + 1]
        tg, a, em, nk = oracle.greedy_accept_request(logits[a0:b0], tokens[a0:b0],
                                                     int(c.lengths.kv[r]))
        assert list(targets[a0:b0].cpu().numpy()) == list(tg)
        assert int(accept[r]) == a and int(new_kv[r]) == nk
        assert list(emitted[r, :a + 1].cpu().numpy()) == list(em)


def test_accept_flags_bad_lengths():
    w = W.SPARSE_BF16.scaled(name="accept_flags", batch=3)
    c = W.make_accept_case(w, 256)
    kv = c.kv_len.clone()
    kv[1] = 2                                          # kv_len < qo_len
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    targets, accept, emitted, new_kv = sdv.greedy_accept(c.logits.to(DEV), c.tokens.to(DEV),
                                                         c.qo_indptr.to(DEV), kv.to(DEV),
                                                         max_qo_len=4, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & sdv._lib.DEVERR_QO_LEN
    assert int(accept[1]) == -1 and int(new_kv[1]) == 2 and bool((emitted[1] == -1).all())
    assert int(accept[0]) >= 0 and int(accept[2]) >= 0
    # the flagged request's rows still get their targets
    ind = c.qo_indptr.numpy()
    tg, _, _, _ = oracle.greedy_accept_request(c.logits.float().numpy()[ind[1]:ind[2]],
                                               c.tokens.numpy()[ind[1]:ind[2]], int(c.lengths.kv[1]))
    assert list(targets[ind[1]:ind[2]].cpu().numpy()) == list(tg)
