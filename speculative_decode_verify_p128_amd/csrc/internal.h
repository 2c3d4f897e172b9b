// Internal launch interface between the C-ABI layer (sdv_api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the API layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sdv.h"

namespace sdv {

// Where a (request, KV head)'s 32-token K/V blocks live.
struct DenseSource {            // P32 sub-page view
  const void* root;             // element 0 of P32 page 0
  const int32_t* sub_offsets;   // [B][2][max_sub_pages], or null: from the block table
  int32_t max_sub_pages;
  int64_t num_sub_pages;        // valid P32 page range from root
  const int32_t* block_table;   // [B][bt_stride] slot ids (when sub_offsets is null)
  int32_t bt_stride;
  int32_t slot_stride;          // the view's index scale
  int32_t num_slots;
};

// P32 page indices of K and V of 32-token block i of request r through the view: from
// the staged offsets, or without them from the block table as the view defines them
// (slot = block_table[r][i / 4], K = 4 * slot_stride * slot + i % 4, V = K + 4).
// False when an index leaves the view (the caller flags it and masks the block out).
__device__ __forceinline__ bool view_pages(const DenseSource& ds, int64_t r, int i, int64_t& xk,
                                           int64_t& xv) {
  if (ds.sub_offsets) {
    const int32_t* offs = ds.sub_offsets + r * 2 * ds.max_sub_pages;
    xk = offs[i];
    xv = offs[ds.max_sub_pages + i];
  } else {
    const int32_t slot = ds.block_table[r * ds.bt_stride + (i >> 2)];
    if (slot < 0 || slot >= ds.num_slots) {
      xk = xv = -1;
      return false;
    }
    xk = 4ll * ds.slot_stride * slot + (i & 3);
    xv = xk + 4;
  }
  return xk >= 0 && xk < ds.num_sub_pages && xv >= 0 && xv < ds.num_sub_pages;
}

struct SparseSource {           // head-major P128 pages + selected page lists
  const void* k;
  const void* v;
  int64_t page_stride;          // elements
  int32_t num_pages;
  const int32_t* block_table;   // [B][bt_stride]
  int32_t bt_stride;
  int32_t max_pages;
  const int32_t* topk_idx;      // [rows][Hkv][top_k]
  int32_t top_k;
  // Selection inside the attention kernels instead of topk_idx (when scores != null):
  // the ladder top-k of scores [rows][Hkv][max_pages], written to topk_out / cnt_out
  // (each nullable) by the workgroups of split 0.
  const float* scores;
  int32_t* topk_out;
  int32_t* cnt_out;
};
// Pages per token the in-kernel selection handles (64 lanes x 16 keys).
constexpr int kFusedTopkMaxPages = 1024;

struct AttnArgs {
  const void* q;
  int32_t q_dt;
  const int32_t* qo_indptr;
  const int32_t* kv_len;
  int32_t B;
  int32_t max_qo_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t kv_dt;
  float k_scale;
  float v_scale;
  float softmax_scale;
  int32_t num_splits;
  float* part_o;                // [splits][rows_cap][Hq][d] when num_splits > 1
  float* part_lse;              // [splits][rows_cap][Hq]
  void* out;
  int32_t out_dt;
  int32_t* dev_err;
  int32_t target_wgs;           // workgroups the GPU holds at once for the chosen kernel
  int32_t order_by_work;        // grid positions take requests longest first (sparse
                                // per-wave launches of more workgroups than the GPU holds)
  int32_t dense_compact;        // dense split-KV grid positions take the (request, KV head,
                                // chunk) pieces that hold blocks, in order (ring kernel)
};

// Bytes per stored element of an sdv_dtype.
__host__ __device__ inline int elem_bytes_of(int32_t dt) {
  return dt == SDV_F32 ? 4 : (dt == SDV_BF16 ? 2 : 1);
}

// Compute units of the current device (cached per device; 0 on error).
inline int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev >= 64) {
    int n = 0;
    return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
  }
  int n = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
  return n;
}

// Workgroups of `kernel` (256 threads, static LDS only) one compute unit holds at once.
template <typename K>
int resident_per_cu(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

hipError_t launch_subpage_offsets(const int32_t* block_table, int32_t B, int32_t max_blocks,
                                  int32_t bt_stride, int32_t slot_stride, int32_t num_slots,
                                  int32_t* sub_offsets, int32_t* dev_err, hipStream_t s);

hipError_t launch_proxy_scores(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                               const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                               int32_t num_q_heads, const sdv_paged_kv& kv,
                               const int32_t* block_table, int32_t max_pages,
                               int32_t bt_stride, float* scores, int32_t* dev_err,
                               hipStream_t s);

hipError_t launch_topk(const float* scores, const int32_t* qo_indptr, const int32_t* kv_len,
                       int32_t B, int32_t max_qo_len, int32_t num_kv_heads,
                       int32_t max_pages, int32_t top_k, int32_t* topk_idx,
                       int32_t* topk_cnt, int32_t* dev_err, hipStream_t s);

// Vector-ALU attention kernels (any supported dtype).
hipError_t launch_attn_dense_valu(const AttnArgs& a, const DenseSource& src, hipStream_t s);
hipError_t launch_attn_sparse_valu(const AttnArgs& a, const SparseSource& src, hipStream_t s);

// Whether the matrix-core attention kernels serve a call: bf16 Q with bf16 or fp8 K/V,
// head_dim 64 or 128, at most 64 query rows (G x max_qo_len) per (request, KV head),
// 16-byte aligned q and out.
inline bool mfma_supported(const AttnArgs& a) {
  const bool aligned = (reinterpret_cast<uintptr_t>(a.q) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(a.out) % 16 == 0);
  return a.q_dt == SDV_BF16 && (a.kv_dt == SDV_BF16 || a.kv_dt == SDV_FP8_E4M3) &&
         (a.head_dim == 64 || a.head_dim == 128) &&
         a.max_qo_len * (a.num_q_heads / a.num_kv_heads) <= 64 && aligned;
}

// 32-token blocks one split of a dense call may hold (the block list a workgroup stages);
// the host rejects calls whose capacity over num_splits exceeds it.
constexpr int kMaxSplitBlocks = 1024;

// Matrix-core attention with an LDS block ring fed by asynchronous global->LDS copies.
hipError_t launch_attn_dense_stream(const AttnArgs& a, const DenseSource& src, hipStream_t s);
hipError_t launch_attn_sparse_stream(const AttnArgs& a, const SparseSource& src, hipStream_t s);

// Matrix-core attention with one block stream per wave (every wave holds all query rows
// and takes every fourth block; same support as above, dense up to 1024 blocks per split).
hipError_t launch_attn_dense_waves(const AttnArgs& a, const DenseSource& src, hipStream_t s);
hipError_t launch_attn_sparse_waves(const AttnArgs& a, const SparseSource& src, hipStream_t s);

// Dense verify attention over ordinary head-major P128 pages and a block table (every
// position below the ladder bound), on the two matrix-core LDS kernels above; `src`
// carries the pools and the block table, topk_idx is unused.
hipError_t launch_attn_paged_waves(const AttnArgs& a, const SparseSource& src, hipStream_t s);
// Dense persistent split-KV (equal block ranges per workgroup over all (request, KV head)
// pairs; num_splits >= 2 partial slots per row, then the combine).  persist_supported
// says whether a call fits it: num_splits >= 2, B <= kPersistMaxRequests,
// ceil(cap_blocks / (num_splits - 1)) <= 1024 and B * Hkv * cap_blocks < 2^31, where
// cap_blocks is the 32-token block capacity of a request.
constexpr int kPersistMaxRequests = 2048;
bool persist_supported(const AttnArgs& a, int64_t cap_blocks);
hipError_t launch_attn_dense_persist(const AttnArgs& a, const DenseSource& src, hipStream_t s);
hipError_t launch_attn_paged_persist(const AttnArgs& a, const SparseSource& src, hipStream_t s);
// The same partition over one LDS block ring per workgroup that runs through the
// boundaries between pieces (same conditions as persist_supported).
hipError_t launch_attn_dense_flat(const AttnArgs& a, const DenseSource& src, hipStream_t s);
hipError_t launch_attn_paged_flat(const AttnArgs& a, const SparseSource& src, hipStream_t s);
hipError_t launch_attn_paged_stream(const AttnArgs& a, const SparseSource& src, hipStream_t s);

// Rows [*row_begin_dev, *row_end_dev) are combined (all rows_cap rows when null).
hipError_t launch_combine(const float* part_o, const float* part_lse, int32_t num_splits,
                          int32_t rows_cap, const int32_t* row_begin_dev,
                          const int32_t* row_end_dev, int32_t num_heads, int32_t head_dim,
                          void* out, int32_t out_dt, float* lse_out, hipStream_t s);

// Ladder KV slot staging: rows [rows][Hkv][d] copied as stored into the paged cache.
hipError_t launch_stage_paged(const void* k_new, const void* v_new, const int32_t* qo_indptr,
                              const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                              const sdv_paged_kv& kv, const int32_t* block_table,
                              int32_t max_pages, int32_t bt_stride, int32_t* dev_err,
                              hipStream_t s);
hipError_t launch_stage_view(const void* k_new, const void* v_new, const int32_t* qo_indptr,
                             const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                             const sdv_subpage_view& view, const int32_t* sub_offsets,
                             int32_t max_sub_pages, int32_t* dev_err, hipStream_t s);

hipError_t launch_copy_descriptors(const void* src, size_t src_bytes, void* dst, size_t dst_bytes,
                                  const sdv_copy_desc* descs, int32_t n, int32_t* dev_err,
                                  hipStream_t s);

// Parts of 1024 16-byte vectors per logits row; the workspace holds a float and an int32
// per (row, part) of B * max_qo_len rows.
int32_t greedy_accept_parts(int32_t vocab, int32_t logits_dt);
hipError_t launch_greedy_accept(const void* logits, int32_t logits_dt, int32_t vocab,
                                const int32_t* tokens, const int32_t* qo_indptr,
                                const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                void* workspace, int32_t* targets, int32_t* accept,
                                int32_t* emitted, int32_t* new_kv_len, int32_t* dev_err,
                                hipStream_t s);

hipError_t launch_fill_u32(void* dst, size_t bytes, uint32_t pattern, hipStream_t s);
hipError_t launch_read_units_probe(const void* base, const int64_t* units, int64_t n_units,
                                   int64_t max_units, int32_t unit_bytes, uint32_t* sink,
                                   int32_t blocks, hipStream_t s);
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                             hipStream_t s);

}  // namespace sdv
