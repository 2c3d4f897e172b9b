"""CPU oracle for multi-token speculative-decoding verify attention.

TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously-correct NumPy code that states
what the verify path computes, one step at a time, in float64 for attention and in
a fixed float32 order for the proxy page scores.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the library path never
does, and it shares no code, header, table or constant with the HIP kernels.

Sources (web pages; cited by title and section in every function):
  [PR18066] "[None][perf] wrap up eagle changes in m3 side branch"
            (NVIDIA/TensorRT-LLM pull 18066): commit fixing the draft view's index
            scale ("view-scale commit"); commit removing code made redundant by the
            native P128 draft view ("dead-code commit").
  [PR17835] "[None][perf] Default Minimax-m3 to unified draft-target kv manager +
            change CI test to GQA eagle head" (NVIDIA/TensorRT-LLM pull 17835):
            sections "Description", "Root causes and fixes" item 2 "Grouped-HND
            draft KV transfer", "Acceptance and accuracy evidence".
  [PR3]     "[TRTLLM-14093][feat] Eagle3 for M3 MSA path + CUDA graphs
            compatibility" (brb-nv/TensorRT-LLM pull 3): the MSA multi-token verify
            commit ("MSA verify commit") and the CUDA-graphs commit.

Readings taken where the pages are silent (each repeated at its function):
  * proxy score: q_t . (sum of the page's keys at positions < bound_t), maximum over
    the query heads of the KV group, ties to the lower page index; unscaled;
    summed in a fixed float32 order (sequential over positions, product without
    fused multiply-add, recursive halving over channels);
  * query heads of KV head h are the contiguous block h*G .. h*G + G - 1;
  * kv_len counts the qo_len verify tokens themselves;
  * fp8 storage is OCP E4M3FN with one float32 scale per tensor;
  * split-KV partitions and their log-sum-exp combine are exact identities.

Pins (tests/test_oracle_*.py) tie each function to something other than itself:
closed forms, brute force, PyTorch's CPU scaled_dot_product_attention in float64,
torch.float8_e4m3fn, coordinate-encoded pools and the pages' own statements.
"""
from .ladder import ladder_bounds, n_valid_pages
from .fp8 import decode_e4m3fn, decode_bf16, decode_store
from .view import (subpage_offsets, gather_subpage_view, gather_hnd, head_slice_contiguous,
                   head_slice_grouped, head_slice_descriptors)
from .attention import attend, dense_verify_request, sparse_verify_request, lse_combine
from .proxy import proxy_scores_request, canonical_dot_f32
from .topk import ladder_topk_request
from .accept import greedy_accept_case, greedy_accept_request, greedy_argmax
from .pipeline import (dense_verify_case, sparse_verify_case, paged_verify_case,
                       request_kv_dense, request_kv_sparse)

__all__ = [
    "ladder_bounds", "n_valid_pages", "decode_e4m3fn", "decode_bf16", "decode_store",
    "subpage_offsets", "gather_subpage_view", "gather_hnd", "head_slice_contiguous",
    "head_slice_grouped", "head_slice_descriptors", "attend", "dense_verify_request", "sparse_verify_request",
    "lse_combine", "proxy_scores_request", "canonical_dot_f32", "ladder_topk_request",
    "dense_verify_case", "sparse_verify_case", "paged_verify_case",
    "request_kv_dense", "request_kv_sparse", "greedy_argmax", "greedy_accept_request",
    "greedy_accept_case",
]
