// Ladder KV slot staging: the verify step writes the K/V of its qo_len new tokens into
// the paged cache ("[TRTLLM-14093][feat] Eagle3 for M3 MSA path + CUDA graphs
// compatibility", MSA verify commit: KV slot staging generalises to the causal ladder).
// Token t of request r lands at logical position kv_len - qo_len + t, across page
// boundaries.  Each request has its own block-table row and its lengths are read on
// the device at every launch, so a correction that shortens one request re-stages it
// at its corrected positions and no other request's pages move (the same commit's
// overlap-correction fix).
//
// One 64-thread workgroup per (request, token slot, KV head): the first d*e/16 lanes
// copy the K row, the next d*e/16 the V row, 16 bytes each; rows are copied as stored.
#include "device.h"
#include "internal.h"

namespace sdv {
namespace {

// Returns false (and flags) when the request's lengths are unusable or the token slot
// is past its qo_len; sets j to the token's logical position otherwise.
__device__ __forceinline__ bool stage_position(const int32_t* qo_indptr, const int32_t* kv_len,
                                               int B, int max_qo_len, int64_t kv_cap, int r,
                                               int t, int h, int& row, int& j, int32_t* dev_err) {
  const int row0 = qo_indptr[r];
  const int qo = qo_indptr[r + 1] - row0;
  const int kv = kv_len[r];
  const bool bad_len = qo < 1 || qo > max_qo_len || kv < qo || row0 < 0 ||
                       static_cast<int64_t>(row0) + qo > static_cast<int64_t>(B) * max_qo_len;
  const bool bad_cap = !bad_len && kv > kv_cap;
  if (bad_len || bad_cap) {
    if (threadIdx.x == 0 && t == 0 && h == 0)
      set_err(dev_err, bad_len ? SDV_DEVERR_QO_LEN : SDV_DEVERR_KV_CAPACITY);
    return false;
  }
  if (t >= qo) return false;
  row = row0 + t;
  j = kv - qo + t;
  return true;
}

__device__ __forceinline__ void copy_row(const char* src, char* dst, int n16, int lane) {
  if (lane < n16)
    reinterpret_cast<uint4*>(dst)[lane] = reinterpret_cast<const uint4*>(src)[lane];
}

__global__ void __launch_bounds__(64) sdv_stage_paged_kernel(
    const char* __restrict__ k_new, const char* __restrict__ v_new, int32_t row_bytes,
    const int32_t* __restrict__ qo_indptr, const int32_t* __restrict__ kv_len, int32_t B,
    int32_t max_qo_len, char* k_pool, char* v_pool, int64_t page_stride_bytes,
    int32_t num_pages, const int32_t* __restrict__ block_table, int32_t bt_stride,
    int32_t max_pages, int32_t* dev_err) {
  const int r = blockIdx.x / max_qo_len;
  const int t = blockIdx.x - r * max_qo_len;
  const int h = blockIdx.y;
  const int Hkv = gridDim.y;
  int row, j;
  if (!stage_position(qo_indptr, kv_len, B, max_qo_len, static_cast<int64_t>(max_pages) * kPage,
                      r, t, h, row, j, dev_err))
    return;
  const int phys = block_table[static_cast<int64_t>(r) * bt_stride + j / kPage];
  if (phys < 0 || phys >= num_pages) {
    if (threadIdx.x == 0) set_err(dev_err, SDV_DEVERR_PAGE_RANGE);
    return;
  }
  const int n16 = row_bytes / 16;
  const int64_t src = (static_cast<int64_t>(row) * Hkv + h) * row_bytes;
  const int64_t dst = phys * page_stride_bytes + (static_cast<int64_t>(h) * kPage + j % kPage) * row_bytes;
  const int lane = threadIdx.x;
  if (lane < n16) copy_row(k_new + src, k_pool + dst, n16, lane);
  else copy_row(v_new + src, v_pool + dst, n16, lane - n16);
}

__global__ void __launch_bounds__(64) sdv_stage_view_kernel(
    const char* __restrict__ k_new, const char* __restrict__ v_new, int32_t row_bytes,
    const int32_t* __restrict__ qo_indptr, const int32_t* __restrict__ kv_len, int32_t B,
    int32_t max_qo_len, char* root, int64_t num_sub_pages,
    const int32_t* __restrict__ sub_offsets, int32_t max_sub_pages, int32_t* dev_err) {
  const int r = blockIdx.x / max_qo_len;
  const int t = blockIdx.x - r * max_qo_len;
  const int h = blockIdx.y;
  const int Hkv = gridDim.y;
  int row, j;
  if (!stage_position(qo_indptr, kv_len, B, max_qo_len, static_cast<int64_t>(max_sub_pages) * kSub,
                      r, t, h, row, j, dev_err))
    return;
  const int32_t* offs = sub_offsets + static_cast<int64_t>(r) * 2 * max_sub_pages;
  const int32_t xk = offs[j / kSub];
  const int32_t xv = offs[max_sub_pages + j / kSub];
  if (xk < 0 || xk + 4 >= num_sub_pages || xv != xk + 4) {
    if (threadIdx.x == 0) set_err(dev_err, SDV_DEVERR_PAGE_RANGE);
    return;
  }
  const int n16 = row_bytes / 16;
  const int64_t src = (static_cast<int64_t>(row) * Hkv + h) * row_bytes;
  const int lane = threadIdx.x;
  const int64_t x = lane < n16 ? xk : xv;
  const int64_t dst = ((x * Hkv + h) * kSub + j % kSub) * row_bytes;
  if (lane < n16) copy_row(k_new + src, root + dst, n16, lane);
  else copy_row(v_new + src, root + dst, n16, lane - n16);
}

}  // namespace

hipError_t launch_stage_paged(const void* k_new, const void* v_new, const int32_t* qo_indptr,
                              const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                              const sdv_paged_kv& kv, const int32_t* block_table,
                              int32_t max_pages, int32_t bt_stride, int32_t* dev_err,
                              hipStream_t s) {
  const int eb = elem_bytes_of(kv.kv_dtype);
  dim3 grid(static_cast<uint32_t>(B) * max_qo_len, kv.num_kv_heads);
  hipLaunchKernelGGL(sdv_stage_paged_kernel, grid, dim3(64), 0, s,
                     reinterpret_cast<const char*>(k_new), reinterpret_cast<const char*>(v_new),
                     kv.head_dim * eb, qo_indptr, kv_len, B, max_qo_len,
                     reinterpret_cast<char*>(const_cast<void*>(kv.k)),
                     reinterpret_cast<char*>(const_cast<void*>(kv.v)), kv.page_stride * eb,
                     kv.num_pages, block_table, bt_stride, max_pages, dev_err);
  return hipGetLastError();
}

hipError_t launch_stage_view(const void* k_new, const void* v_new, const int32_t* qo_indptr,
                             const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                             const sdv_subpage_view& view, const int32_t* sub_offsets,
                             int32_t max_sub_pages, int32_t* dev_err, hipStream_t s) {
  const int eb = elem_bytes_of(view.kv_dtype);
  dim3 grid(static_cast<uint32_t>(B) * max_qo_len, view.num_kv_heads);
  hipLaunchKernelGGL(sdv_stage_view_kernel, grid, dim3(64), 0, s,
                     reinterpret_cast<const char*>(k_new), reinterpret_cast<const char*>(v_new),
                     view.head_dim * eb, qo_indptr, kv_len, B, max_qo_len,
                     reinterpret_cast<char*>(const_cast<void*>(view.k_root)), view.num_sub_pages,
                     sub_offsets, max_sub_pages, dev_err);
  return hipGetLastError();
}

}  // namespace sdv
