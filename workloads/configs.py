"""Workload shapes for the speculative-decoding verify step.

Five frozen workload descriptions. Each gives the batch, how the per-request query
length (qo_len = 1 + draft_len) and KV length are drawn, the head geometry, the
storage dtype of K/V and Q, the top-k page budget of the sparse layer and the pool
geometry of the dense draft layer.  Nothing here computes anything of the method:
the shapes only.

Page geometry facts come from the pages:
  * target KV uses 128-token physical pages and the Eagle3 drafter consumes
    32-token pages through a non-owning sub-page view (PR #17835 "Default
    Minimax-m3 to unified draft-target kv manager ...", section Description);
  * the draft layer's flat pool puts slot s's K page at s * stride and its V page at
    s * stride + 1, counted from the draft layer's own K page (PR #18066 "wrap up
    eagle changes in m3 side branch", commit that fixes the draft view's index
    scale);
  * qo_len = 1 + draft_len with draft_len 3 (PR #3 "Eagle3 for M3 MSA path + CUDA
    graphs compatibility", MSA multi-token verify and CUDA-graphs commits).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple

PAGE = 128      # physical page, tokens
SUB_PAGE = 32   # draft-view sub-page, tokens


@dataclass(frozen=True)
class VerifyWorkload:
    name: str
    batch: int
    # qo_len: fixed value, or ("uniform", lo, hi) inclusive
    qo: object
    # kv_len: ("list", (a, b, ...)), ("uniform", lo, hi), ("fixed", n),
    #         ("lognormal", median, sigma, lo, hi, crossing_fraction)
    kv: Tuple
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str            # "f32" | "bf16" | "fp8"
    q_dtype: str             # "f32" | "bf16"
    values: str              # "int4" (integers in [-4, 4]) | "normal" (N(0, 1))
    top_k: int
    num_splits: int = 1
    slot_stride: int = 8     # dense draft pool: pages per slot
    root_page: int = 6       # in-slot page of the draft layer's K page (V at +1)
    pool_index_scale: int = 8  # pool-level page-index scale; the view ignores it
    kv_capacity: Optional[int] = None  # tokens a block table can address
    spare_pages: int = 8

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def capacity_tokens(self) -> int:
        if self.kv_capacity is not None:
            return self.kv_capacity
        kind = self.kv[0]
        if kind == "list":
            return max(self.kv[1])
        if kind == "uniform":
            return self.kv[2]
        if kind == "fixed":
            return self.kv[1]
        if kind == "lognormal":
            return self.kv[4]
        raise ValueError(kind)

    def max_pages(self) -> int:
        return -(-self.capacity_tokens() // PAGE)

    def max_qo(self) -> int:
        return self.qo if isinstance(self.qo, int) else self.qo[2]

    def scaled(self, **kw) -> "VerifyWorkload":
        return replace(self, **kw)


# 1. Tiny full pipeline in fp32 with integer values (every score exact in fp32).
TINY_FP32 = VerifyWorkload(
    name="tiny_fp32", batch=2, qo=4, kv=("list", (300, 517)),
    num_q_heads=8, num_kv_heads=2, head_dim=64, kv_dtype="f32", q_dtype="f32",
    values="int4", top_k=2, num_splits=1, slot_stride=2, root_page=0,
    pool_index_scale=2)

# 2. Dense GQA draft layer through the 32-token sub-page view, bf16.
DENSE_BF16 = VerifyWorkload(
    name="dense_bf16", batch=32, qo=4, kv=("uniform", 1024, 8192),
    num_q_heads=64, num_kv_heads=4, head_dim=128, kv_dtype="bf16", q_dtype="bf16",
    values="normal", top_k=16, num_splits=6, slot_stride=8, root_page=6,
    pool_index_scale=8)

# 3. Block-sparse target layer, bf16.
SPARSE_BF16 = VerifyWorkload(
    name="sparse_bf16", batch=64, qo=4, kv=("uniform", 4096, 32768),
    num_q_heads=16, num_kv_heads=4, head_dim=128, kv_dtype="bf16", q_dtype="bf16",
    values="normal", top_k=16, num_splits=1)

# 4. Long-context sparse verify with fp8 e4m3 K/V and a 16-way split-KV.
LONG_FP8 = VerifyWorkload(
    name="long_fp8", batch=8, qo=4, kv=("fixed", 131072),
    num_q_heads=16, num_kv_heads=4, head_dim=128, kv_dtype="fp8", q_dtype="bf16",
    values="normal", top_k=64, num_splits=16)

# 5. Ragged mixed batch through both paths.
RAGGED_MIXED = VerifyWorkload(
    name="ragged_mixed", batch=256, qo=("uniform", 1, 8),
    kv=("lognormal", 2048, 1.0, 64, 65536, 0.25),
    num_q_heads=16, num_kv_heads=4, head_dim=128, kv_dtype="bf16", q_dtype="bf16",
    values="normal", top_k=16, num_splits=2, slot_stride=8, root_page=6,
    pool_index_scale=8)

# 6. The target model's dense layers (ladder mask over every page) on the sparse
#    workload's geometry and lengths: ordinary head-major P128 pages, bf16.
PAGED_BF16 = VerifyWorkload(
    name="paged_bf16", batch=64, qo=4, kv=("uniform", 4096, 32768),
    num_q_heads=16, num_kv_heads=4, head_dim=128, kv_dtype="bf16", q_dtype="bf16",
    values="normal", top_k=16, num_splits=3)

ALL = (TINY_FP32, DENSE_BF16, SPARSE_BF16, LONG_FP8, RAGGED_MIXED, PAGED_BF16)
BY_NAME = {w.name: w for w in ALL}
