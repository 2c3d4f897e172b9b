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
// Each round reduces the lanes' cached maxima across the wave — a rotate-and-max inside
// each 16-lane row (DPP row rotations, no LDS traffic), then the four row maxima read
// into scalar registers — and the owning lane retires the key and refreshes its cache.
#include "device.h"
#include "internal.h"

namespace sdv {

// Lane l's 64-bit value of lane (l - N) mod 16 of its row: DPP row_ror:N on each half.
template <int N>
__device__ __forceinline__ uint64_t row_rotate(uint64_t v) {
  constexpr int kRowRor = 0x120;   // DPP row_ror:n, n = 1 .. 15
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(
      static_cast<int>(static_cast<uint32_t>(v)), kRowRor + N, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(
      static_cast<int>(static_cast<uint32_t>(v >> 32)), kRowRor + N, 0xF, 0xF, false));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t lane_value(uint64_t v, int lane) {
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), lane);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

// Maximum of v over the wave, the same in every lane.
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
  v = umax64(v, row_rotate<1>(v));
  v = umax64(v, row_rotate<2>(v));
  v = umax64(v, row_rotate<4>(v));
  v = umax64(v, row_rotate<8>(v));     // every lane of a row holds the row's maximum
  return umax64(umax64(lane_value(v, 0), lane_value(v, 16)),
                umax64(lane_value(v, 32), lane_value(v, 48)));
}

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

  uint64_t keys[ITEMS];
  uint64_t best = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int p = lane + kWave * i;
    keys[i] = p < n ? (static_cast<uint64_t>(ordered_key(srow[p])) << 32) |
                          static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(p))
                    : 0ull;
    best = keys[i] > best ? keys[i] : best;
  }
  const int k_eff = top_k < n ? top_k : n;
  int32_t* out = topk_idx + (row * Hkv + h) * top_k;
  for (int k = 0; k < k_eff; ++k) {
    const uint64_t m = wave_max64(best);
    if (best == m) {                   // keys are unique: exactly one lane owns m
      uint64_t nb = 0;
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        keys[i] = keys[i] == m ? 0ull : keys[i];
        nb = keys[i] > nb ? keys[i] : nb;
      }
      best = nb;
    }
    if (lane == 0) out[k] = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(m));
  }
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
