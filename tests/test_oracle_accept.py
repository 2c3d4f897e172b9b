"""Pins of the greedy-acceptance oracle: a hand-worked example, the argmax against
NumPy's library routines (ties to the lowest index, NaN skipped), invariants on seeded
cases, and an independent vectorised formulation of the accepted prefix."""
import numpy as np
import torch

import oracle
import workloads as W


def test_hand_worked_example():
    # verify input [5, 7, 2, 9]; the target's greedy tokens after each row: 7, 2, 3, 1.
    # d1 = 7 matches, d2 = 2 matches, d3 = 9 != 3: two drafts accepted, then the bonus
    # token 3; the cache keeps 5, 7, 2 of the four verify tokens.
    vocab = 10
    logits = np.zeros((4, vocab))
    for t, tgt in enumerate((7, 2, 3, 1)):
        logits[t, tgt] = 1.0
    targets, a, emitted, new_kv = oracle.greedy_accept_request(logits, np.array([5, 7, 2, 9]), 100)
    assert list(targets) == [7, 2, 3, 1] and a == 2
    assert list(emitted) == [7, 2, 3] and new_kv == 99


def test_decode_row_and_full_acceptance():
    logits = np.eye(6)[[4]]
    t, a, em, kv = oracle.greedy_accept_request(logits, np.array([1]), 10)
    assert a == 0 and list(em) == [4] and kv == 10          # qo_len = 1: plain decode
    logits = np.eye(6)[[1, 2, 3, 5]]
    t, a, em, kv = oracle.greedy_accept_request(logits, np.array([0, 1, 2, 3]), 50)
    assert a == 3 and list(em) == [1, 2, 3, 5] and kv == 50  # every draft accepted


def test_argmax_matches_numpy_ties_and_nan():
    rng = np.random.default_rng(3)
    x = rng.integers(-3, 4, size=(200, 37)).astype(np.float64)   # many equal maxima
    for row in x:
        assert oracle.greedy_argmax(row) == int(np.argmax(row))
    x[:, ::5] = np.nan
    for row in x:
        assert oracle.greedy_argmax(row) == int(np.nanargmax(row))
    assert oracle.greedy_argmax(np.full(5, np.nan)) == -1


def test_seeded_cases_invariants_and_vectorised_prefix():
    for w, dt in ((W.SPARSE_BF16, torch.bfloat16), (W.RAGGED_MIXED, torch.float32)):
        c = W.make_accept_case(w, 512, dtype=dt, nan_rows=0.05)
        logits = c.logits.float().numpy()
        tokens = c.tokens.numpy()
        ind = c.qo_indptr.numpy()
        res = oracle.greedy_accept_case(logits, tokens, ind, c.lengths.kv)
        for r in range(w.batch):
            a0, b0 = ind[r], ind[r + 1]
            qo, a = b0 - a0, int(res["accept"][r])
            tg = res["targets"][a0:b0]
            # independent formulation: accepted = length of the all-true prefix of matches
            match = tokens[a0 + 1:b0] == tg[:qo - 1]
            assert a == int(np.cumprod(match).sum())
            assert 0 <= a <= qo - 1
            em = res["emitted"][r]
            assert list(em[:a]) == list(tokens[a0 + 1:a0 + 1 + a]) and em[a] == tg[a]
            assert np.all(em[a + 1:] == -1)
            assert res["new_kv"][r] == c.lengths.kv[r] - qo + 1 + a
