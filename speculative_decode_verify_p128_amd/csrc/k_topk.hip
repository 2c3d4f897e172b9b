// Per-token ladder-bounded top-k page selection.
//
// "[TRTLLM-14093][feat] Eagle3 for M3 MSA path + CUDA graphs compatibility", MSA
// multi-token verify commit: top-k gets each token's own ladder valid-page count, so a
// draft token cannot select pages past its own attend bound.  Order: score
// descending, then page index ascending (ties go to the lower page); output in rank
// order, -1 padded.
//
// One wave per (token row, KV head).  Lane l holds pages l, l + 64, ... of the token's
// n_valid pages as 64-bit keys (order-preserving score bits << 32 | ~page), so one
// unsigned maximum picks the best score and, among equal scores, the lowest page.
// Each round takes the wave maximum of the lanes' cached score words (DPP row rotations,
// then the four row maxima in scalar registers), settles equal scores on the page word
// only when a ballot shows a tie, and the owning lane retires the key and refreshes its
// cache (wave_ladder_topk, shared with the selection inside the sparse attention
// kernels).
#include "device.h"
#include "internal.h"

namespace sdv {

template <int ITEMS>
__global__ void __launch_bounds__(64) sdv_topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ qo_indptr,
    const int32_t* __restrict__ kv_len, int32_t B, int32_t max_qo_len, int32_t Hkv,
    int32_t max_pages, int32_t top_k, int32_t* __restrict__ topk_idx,
    int32_t* __restrict__ topk_cnt, int32_t* dev_err) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int r = blockIdx.z;
  const int lane = threadIdx.x;
  const int row0 = qo_indptr[r];
  const int qo = qo_indptr[r + 1] - row0;
  const int kv = kv_len[r];
  const bool bad_len = qo < 1 || qo > max_qo_len || kv < qo || row0 < 0 ||
                       static_cast<int64_t>(row0) + qo > static_cast<int64_t>(B) * max_qo_len;
  const bool bad_cap = !bad_len && static_cast<int64_t>(kv) > static_cast<int64_t>(max_pages) * kPage;
  if (bad_len || bad_cap) {
    if (lane == 0 && t == 0 && h == 0)
      set_err(dev_err, bad_len ? SDV_DEVERR_QO_LEN : SDV_DEVERR_KV_CAPACITY);
    return;
  }
  if (t >= qo) return;
  const int bound = kv - qo + t + 1;
  const int n = (bound + kPage - 1) / kPage;
  const int64_t row = row0 + t;
  const float* srow = scores + (row * Hkv + h) * max_pages;

  int32_t* out = topk_idx + (row * Hkv + h) * top_k;
  const int k_eff = wave_ladder_topk<ITEMS>(srow, n, top_k, lane, [&](int k, int page) {
    if (lane == 0) out[k] = page;
  });
  for (int k = k_eff + lane; k < top_k; k += kWave) out[k] = -1;
  if (topk_cnt && lane == 0) topk_cnt[row * Hkv + h] = k_eff;
}

hipError_t launch_topk(const float* scores, const int32_t* qo_indptr, const int32_t* kv_len,
                       int32_t B, int32_t max_qo_len, int32_t num_kv_heads, int32_t max_pages,
                       int32_t top_k, int32_t* topk_idx, int32_t* topk_cnt, int32_t* dev_err,
                       hipStream_t s) {
  dim3 grid(max_qo_len, num_kv_heads, B);
  const int items = (max_pages + kWave - 1) / kWave;
#define SDV_TOPK_CASE(N)                                                                     \
  if (items <= N) {                                                                          \
    hipLaunchKernelGGL(sdv_topk_kernel<N>, grid, dim3(kWave), 0, s, scores, qo_indptr, kv_len, \
                       B, max_qo_len, num_kv_heads, max_pages, top_k, topk_idx, topk_cnt,    \
                       dev_err);                                                             \
    return hipGetLastError();                                                                \
  }
  SDV_TOPK_CASE(1)
  SDV_TOPK_CASE(2)
  SDV_TOPK_CASE(4)
  SDV_TOPK_CASE(8)
  SDV_TOPK_CASE(16)
  SDV_TOPK_CASE(32)
  SDV_TOPK_CASE(64)
#undef SDV_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace sdv
