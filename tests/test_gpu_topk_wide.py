"""GPU parity of the ladder top-k over wide page tables (more than 256 pages: with a large
top_k one workgroup per (token, KV head) finds the k-th largest key and sorts the
selection, with a small one the wave kernel runs; both are exercised here):
indices and counts bit-exact with the oracle's selection, on float scores, on integer
scores with many exact ties and signed zeros, for top_k up to 1024 and for tokens with
fewer valid pages than top_k."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decode_verify_p128_amd as sdv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


def _run(kv, qo, max_pages, top_k, scores_np, Hkv):
    ind = np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)
    idx, cnt = sdv.ladder_topk_pages(torch.from_numpy(scores_np).to(DEV),
                                     torch.from_numpy(ind).to(DEV),
                                     torch.from_numpy(np.asarray(kv, dtype=np.int32)).to(DEV),
                                     max_qo_len=int(max(qo)), top_k=top_k, want_count=True)
    torch.cuda.synchronize()
    got, gcnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for r in range(len(kv)):
        a, b = ind[r], ind[r + 1]
        e, c = oracle.ladder_topk_request(scores_np[a:b], int(kv[r]), top_k)
        assert np.array_equal(got[a:b], e.astype(np.int32)), f"request {r}"
        assert np.array_equal(gcnt[a:b], c.astype(np.int32)), f"request {r}"


@pytest.mark.parametrize("max_pages,top_k", [(257, 16), (1024, 64), (1024, 1), (2000, 300),
                                             (4096, 1024), (4096, 64)])
@pytest.mark.parametrize("kind", ["float", "int_ties"])
def test_wide_topk_bit_exact(max_pages, top_k, kind):
    rng = np.random.default_rng(max_pages * 7 + top_k)
    Hkv, B, max_qo = 2, 3, 4
    # one request at capacity, one with fewer valid pages than top_k, one crossing a page
    kv = np.array([max_pages * 128, max(4, min(top_k, 40) * 128 - 300), 300 * 128 + 2])
    kv = np.minimum(kv, max_pages * 128)
    qo = np.array([4, 4, 3])
    rows = B * max_qo
    if kind == "float":
        scores = rng.standard_normal((rows, Hkv, max_pages)).astype(np.float32)
    else:
        scores = rng.integers(-3, 4, size=(rows, Hkv, max_pages)).astype(np.float32)
        zeros = scores == 0
        scores[zeros] = np.where(rng.random(zeros.sum()) < 0.5, -0.0, 0.0)
    _run(kv, qo, max_pages, top_k, scores, Hkv)


def test_wide_topk_equal_scores_everywhere():
    """Every score equal: the selection is the lowest pages, in index order."""
    max_pages, top_k = 1500, 200
    kv = np.array([max_pages * 128, 130])
    qo = np.array([4, 2])
    scores = np.full((8, 1, max_pages), 2.5, dtype=np.float32)
    _run(kv, qo, max_pages, top_k, scores, 1)
