"""MI355X-native speculative-decoding verify attention (HIP kernels for gfx950 behind a
C ABI, see include/sdv.h).  The PyTorch binding passes tensors' device pointers and
the current stream; nothing here computes on the host."""
from .api import (PagedKV, SubpageView, alloc_workspace, copy_descriptors, dtype_code, fill_u32,
                  greedy_accept, greedy_accept_workspace_bytes, hnd_head_slice_descriptors,
                  kv_subpage_view_init, ladder_topk_pages, lse_combine, proxy_page_scores,
                  read_probe, read_units_probe, stage_verify_kv_paged, stage_verify_kv_view,
                  verify_attention_dense, verify_attention_dense_view,
                  verify_attention_dense_view_noalloc, verify_attention_paged,
                  verify_attention_sparse, verify_attention_sparse_select, workspace_bytes)
from ._lib import (FAMILY_AUTO, FAMILY_FLAT, FAMILY_PERSIST, FAMILY_RING, FAMILY_VALU,
                   FAMILY_WAVES, LIB_PATH, XCHECK_LIB_PATH, SdvError, load, load_xcheck)

__all__ = [
    "PagedKV", "SubpageView", "alloc_workspace", "copy_descriptors", "dtype_code", "fill_u32",
    "greedy_accept", "greedy_accept_workspace_bytes", "hnd_head_slice_descriptors",
    "kv_subpage_view_init", "ladder_topk_pages", "lse_combine", "proxy_page_scores",
    "read_probe", "read_units_probe", "stage_verify_kv_paged", "stage_verify_kv_view",
    "verify_attention_dense", "verify_attention_dense_view",
    "verify_attention_dense_view_noalloc", "verify_attention_paged",
    "verify_attention_sparse", "verify_attention_sparse_select", "workspace_bytes",
    "FAMILY_AUTO", "FAMILY_FLAT", "FAMILY_PERSIST", "FAMILY_RING", "FAMILY_VALU",
    "FAMILY_WAVES", "LIB_PATH", "XCHECK_LIB_PATH", "SdvError", "load", "load_xcheck",
]
