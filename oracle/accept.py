"""Greedy acceptance of draft tokens after the verify step (mechanics only; the pages'
acceptance statistics need trained models).

[PR17835] "Acceptance and accuracy evidence": acceptance is measured under greedy
decoding, reported as acceptance rate and mean acceptance length.  [PR3] MSA verify
commit: the verify batch is qo_len = 1 + draft_len tokens per request.

Reading (the plainest one the pages support, stated here because they give no code):
  * row t of a request holds its t-th verify input token: row 0 the last accepted
    token, rows 1 .. qo_len - 1 the draft tokens d_1 .. d_{qo_len - 1};
  * the target's greedy token after row t is argmax of that row's logits, ties to the
    lowest vocabulary index, NaN never selected (a row of NaN only gives -1);
  * draft d_{t+1} is accepted while it equals the target token after row t for every
    earlier row; a = the number of accepted drafts (0 .. qo_len - 1);
  * the step emits d_1 .. d_a and the bonus token, the target after row a: a + 1 tokens
    (the acceptance length), so acceptance rate = a / (qo_len - 1);
  * the cache keeps the verify tokens up to and including d_a: the corrected kv_len is
    kv_len - qo_len + 1 + a (the bonus token is the next step's first verify token).
"""
import numpy as np


def greedy_argmax(logits_row: np.ndarray) -> int:
    """Index of the largest value, lowest index on ties, NaN never selected (-1 if the
    row holds only NaN)."""
    x = np.asarray(logits_row, dtype=np.float64)
    best, arg = -np.inf, -1
    for i, v in enumerate(x):
        if np.isnan(v):
            continue
        if arg < 0 or v > best:
            best, arg = v, i
    return arg


def greedy_accept_request(logits: np.ndarray, tokens: np.ndarray, kv_len: int):
    """logits [qo, vocab] (values), tokens [qo] int.  Returns (targets [qo], a,
    emitted [a + 1], new_kv_len)."""
    qo = logits.shape[0]
    targets = np.array([greedy_argmax(logits[t]) for t in range(qo)], dtype=np.int64)
    a = 0
    while a < qo - 1 and tokens[a + 1] == targets[a]:
        a += 1
    emitted = np.concatenate([np.asarray(tokens[1:a + 1], dtype=np.int64), targets[a:a + 1]])
    return targets, a, emitted, kv_len - qo + 1 + a


def greedy_accept_case(logits, tokens, qo_indptr, kv_len):
    """Whole batch: targets [rows], accept [B], emitted [B, max_qo] (-1 padded),
    new_kv [B]."""
    B = len(kv_len)
    max_qo = int(np.max(np.diff(qo_indptr))) if B else 1
    rows = int(qo_indptr[-1]) if B else 0
    targets = np.full(rows, -1, dtype=np.int64)
    accept = np.zeros(B, dtype=np.int64)
    emitted = np.full((B, max_qo), -1, dtype=np.int64)
    new_kv = np.zeros(B, dtype=np.int64)
    for r in range(B):
        a0, b0 = int(qo_indptr[r]), int(qo_indptr[r + 1])
        t, a, em, nk = greedy_accept_request(logits[a0:b0], tokens[a0:b0], int(kv_len[r]))
        targets[a0:b0] = t
        accept[r] = a
        emitted[r, :a + 1] = em
        new_kv[r] = nk
    return {"targets": targets, "accept": accept, "emitted": emitted, "new_kv": new_kv}
