"""Verify attention in float64: dense under the ladder, sparse over selected pages, and
the split-KV log-sum-exp combine.

[PR3] MSA verify commit: each verify token t attends kv_len - qo_len + t + 1
positions; the sparse GQA pass attends only the pages its top-k selected; dense
target layers use a ladder mask that equals the old single-token math at qo_len = 1.
[PR17835] Description: the Eagle3 drafter's dense attention reads its KV through the
P32 sub-page view.  [PR18066] (opening commit): the drafter is GQA with 4 KV heads.

Readings: softmax scale is a caller constant (1/sqrt(head_dim) in the workloads);
query heads of KV head h are h*G .. h*G + G - 1; scores and values use the decoded
stored values times the per-tensor scale; accumulation is float64 here.
"""
import numpy as np

from .ladder import ladder_bounds

PAGE = 128


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray, scale: float):
    """Softmax attention of rows q [R, d] over keys k/v [n, d] restricted by the boolean
    mask allowed [R, n].  Returns (out [R, d], lse [R]) with lse the natural log of
    sum_j exp(scale * q.k_j) over allowed j; a row with nothing allowed gets out = 0
    and lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    R, d = q.shape
    out = np.zeros((R, v.shape[1]), dtype=np.float64)
    lse = np.full(R, -np.inf)
    if k.shape[0] == 0:
        return out, lse
    s = scale * (q @ np.asarray(k, dtype=np.float64).T)            # [R, n]
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1)
    live = ~(m == -np.inf)            # NaN stays live so that it propagates
    if not live.any():
        return out, lse
    e = np.zeros_like(s)
    e[live] = np.exp(s[live] - m[live, None])
    l = e.sum(axis=1)
    # Each row sums over its own allowed positions only, so storage a row may not
    # see (stale or foreign, possibly NaN) never enters its output.
    v = np.asarray(v, dtype=np.float64)
    for r in np.nonzero(live)[0]:
        sel = allowed[r]
        out[r] = (e[r, sel] @ v[sel]) / l[r]
    lse[live] = m[live] + np.log(l[live])
    return out, lse


def _rows_of_head(q_req: np.ndarray, h: int, G: int) -> np.ndarray:
    """Rows (t, g) -> q[t, h*G + g] as an array [qo * G, d], row index t * G + g."""
    qo, _, d = q_req.shape
    return q_req[:, h * G:(h + 1) * G, :].reshape(qo * G, d)


def dense_verify_request(q_req, k_seq, v_seq, kv_len: int, scale: float, return_lse=False):
    """One request of dense verify attention.

    q_req [qo, Hq, d]; k_seq, v_seq [kv_len, Hkv, d] (values, already scaled).
    Token t sees positions j < kv_len - qo + t + 1.  Returns out [qo, Hq, d]."""
    qo, Hq, d = q_req.shape
    Hkv = k_seq.shape[1]
    G = Hq // Hkv
    bound = ladder_bounds(kv_len, qo)
    pos = np.arange(kv_len)
    allowed_t = pos[None, :] < bound[:, None]                       # [qo, kv]
    allowed = np.repeat(allowed_t, G, axis=0)                       # rows t*G + g
    out = np.zeros((qo, Hq, d))
    lse = np.zeros((qo, Hq))
    for h in range(Hkv):
        o, l = attend(_rows_of_head(q_req, h, G), k_seq[:, h, :], v_seq[:, h, :], allowed, scale)
        out[:, h * G:(h + 1) * G, :] = o.reshape(qo, G, d)
        lse[:, h * G:(h + 1) * G] = l.reshape(qo, G)
    return (out, lse) if return_lse else out


def sparse_verify_request(q_req, k_seq, v_seq, kv_len: int, topk_idx, scale: float,
                          page: int = PAGE, return_lse=False):
    """One request of block-sparse verify attention.

    topk_idx [qo, Hkv, K]: request-local page numbers chosen by token t for KV head h
    (-1 = unused).  Token t, head h sees position j iff j < bound_t and page j // 128
    is among its chosen pages."""
    qo, Hq, d = q_req.shape
    Hkv = k_seq.shape[1]
    G = Hq // Hkv
    bound = ladder_bounds(kv_len, qo)
    pos = np.arange(kv_len)
    out = np.zeros((qo, Hq, d))
    lse = np.zeros((qo, Hq))
    for h in range(Hkv):
        allowed_t = np.zeros((qo, kv_len), dtype=bool)
        for t in range(qo):
            chosen = [int(p) for p in topk_idx[t, h] if p >= 0]
            in_sel = np.isin(pos // page, chosen)
            allowed_t[t] = in_sel & (pos < bound[t])
        allowed = np.repeat(allowed_t, G, axis=0)
        o, l = attend(_rows_of_head(q_req, h, G), k_seq[:, h, :], v_seq[:, h, :], allowed, scale)
        out[:, h * G:(h + 1) * G, :] = o.reshape(qo, G, d)
        lse[:, h * G:(h + 1) * G] = l.reshape(qo, G)
    return (out, lse) if return_lse else out


def lse_combine(partial_out: np.ndarray, partial_lse: np.ndarray):
    """Merge S partial attentions over disjoint key sets.

    partial_out [S, R, d] (each normalised over its own keys), partial_lse [S, R].
    LSE = log sum_s exp(lse_s); out = sum_s exp(lse_s - LSE) * out_s.  Partials with
    lse = -inf carry no keys and get weight 0; a row with none gets out 0, LSE -inf."""
    po = np.asarray(partial_out, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    m = pl.max(axis=0)
    live = np.isfinite(m)
    w = np.zeros_like(pl)
    w[:, live] = np.exp(pl[:, live] - m[None, live])
    tot = w.sum(axis=0)
    LSE = np.full(pl.shape[1], -np.inf)
    LSE[live] = m[live] + np.log(tot[live])
    out = np.zeros(po.shape[1:])
    safe = np.where(w[:, :, None] > 0, po, 0.0)
    out[live] = (w[:, live, None] * safe[:, live]).sum(axis=0) / tot[live, None]
    return out, LSE
