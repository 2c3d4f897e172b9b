// Greedy acceptance of the draft tokens after the verify step.  Acceptance under greedy
// decoding is what "[None][perf] Default Minimax-m3 to unified draft-target kv manager
// ...", Acceptance and accuracy evidence, measures; the verify batch holds qo_len =
// 1 + draft_len tokens per request ("[TRTLLM-14093][feat] Eagle3 for M3 MSA path + CUDA
// graphs compatibility", MSA verify commit).
//
//   1. sdv_argmax_kernel: one 1024-thread workgroup per verify row streams its vocab
//      logits with 16-byte non-temporal loads, 16 in flight per thread (HBM-bound):
//      the row's largest non-NaN value, then the lowest index holding it, from the same
//      registers — the target's greedy token after that row (ties to the lowest index,
//      NaN never selected).
//   2. sdv_accept_kernel: one thread per request takes the longest prefix of drafts
//      equal to the targets of the rows before them, emits them and the bonus target,
//      and writes the corrected kv_len (kv_len - qo_len + 1 + accepted).
#include <climits>

#include "device.h"
#include "internal.h"

namespace sdv {
namespace {

typedef unsigned int u32x4_acc __attribute__((ext_vector_type(4)));

constexpr int kArgmaxThreads = 1024;
constexpr int kArgmaxUnroll = 16;     // 16-byte loads in flight per thread

// Decoded logits of one 16-byte load.
template <int DT>
__device__ __forceinline__ void decode16(const u32x4_acc& w, float (&x)[16 / (DT == SDV_F32 ? 4 : 2)]) {
  if constexpr (DT == SDV_F32) {
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(w[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
}

// Two passes over the row, the loaded logits kept in registers between them: the row's
// largest value M (fmaxf skips NaN; a row of NaN leaves M = -inf), reduced over the
// workgroup, then the lowest index whose logit equals M (none when the row holds only
// NaN).  This is exactly the argmax with ties to the lowest index and NaN never chosen.
template <int DT>
__global__ void __launch_bounds__(kArgmaxThreads) sdv_argmax_kernel(
    const char* __restrict__ logits, int32_t vocab, const int32_t* __restrict__ qo_indptr,
    int32_t B, int32_t* __restrict__ targets) {
  constexpr int EB = DT == SDV_F32 ? 4 : 2;
  constexpr int PER = 16 / EB;                 // elements per 16-byte load
  constexpr int NW = kArgmaxThreads / kWave;
  __shared__ float s_max[NW];
  __shared__ int s_idx[NW];
  const int row = blockIdx.x;
  if (row >= qo_indptr[B]) return;
  const u32x4_acc* base = reinterpret_cast<const u32x4_acc*>(logits + static_cast<int64_t>(row) * vocab * EB);
  const int nvec = vocab / PER;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY;
  int best = INT_MAX;
  // rows up to kArgmaxThreads * kArgmaxUnroll vectors: one register batch, both passes
  // from registers; longer rows: the batches of pass 2 are loaded again
  constexpr int STEP = kArgmaxThreads * kArgmaxUnroll;
  u32x4_acc w[kArgmaxUnroll];
  for (int pass = 0; pass < 2; ++pass) {
    for (int v0 = threadIdx.x; v0 - static_cast<int>(threadIdx.x) < nvec; v0 += STEP) {
      if (pass == 0 || nvec > STEP) {
#pragma unroll
        for (int u = 0; u < kArgmaxUnroll; ++u) {
          const int v = v0 + u * kArgmaxThreads;
          w[u] = v < nvec ? __builtin_nontemporal_load(base + v) : u32x4_acc{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < kArgmaxUnroll; ++u) {
        const int v = v0 + u * kArgmaxThreads;
        if (v >= nvec) continue;
        float x[PER];
        decode16<DT>(w[u], x);
        if (pass == 0) {
#pragma unroll
          for (int k = 0; k < PER; ++k) m = fmaxf(m, x[k]);
        } else {
#pragma unroll
          for (int k = 0; k < PER; ++k)
            if (x[k] == m && v * PER + k < best) best = v * PER + k;
        }
      }
    }
    if (pass == 0) {
      // workgroup maximum
      m = wave_max(m);
      if (lane == 0) s_max[wave] = m;
      __syncthreads();
      m = s_max[0];
#pragma unroll
      for (int k = 1; k < NW; ++k) m = fmaxf(m, s_max[k]);
    }
  }
  // workgroup minimum of the indices holding the maximum (an all-NaN row keeps m = -inf,
  // which no NaN equals, so best stays INT_MAX)
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) best = min(best, __shfl_xor(best, off, kWave));
  if (lane == 0) s_idx[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    int b = s_idx[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) b = min(b, s_idx[k]);
    targets[row] = b == INT_MAX ? -1 : b;
  }
}

__global__ void __launch_bounds__(64) sdv_accept_kernel(
    const int32_t* __restrict__ targets, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ qo_indptr, const int32_t* __restrict__ kv_len, int32_t B,
    int32_t max_qo_len, int32_t* __restrict__ accept, int32_t* __restrict__ emitted,
    int32_t* __restrict__ new_kv_len, int32_t* dev_err) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= B) return;
  const int row0 = qo_indptr[r];
  const int qo = qo_indptr[r + 1] - row0;
  const int kv = kv_len[r];
  int32_t* em = emitted + static_cast<int64_t>(r) * max_qo_len;
  if (qo < 1 || qo > max_qo_len || kv < qo || row0 < 0 ||
      static_cast<int64_t>(row0) + qo > static_cast<int64_t>(B) * max_qo_len) {
    set_err(dev_err, SDV_DEVERR_QO_LEN);
    accept[r] = -1;
    new_kv_len[r] = kv;
    for (int t = 0; t < max_qo_len; ++t) em[t] = -1;
    return;
  }
  int a = 0;
  while (a < qo - 1 && tokens[row0 + a + 1] == targets[row0 + a]) ++a;
  for (int t = 0; t < max_qo_len; ++t)
    em[t] = t < a ? tokens[row0 + t + 1] : (t == a ? targets[row0 + a] : -1);
  accept[r] = a;
  new_kv_len[r] = kv - qo + 1 + a;
}

}  // namespace

hipError_t launch_greedy_accept(const void* logits, int32_t logits_dt, int32_t vocab,
                                const int32_t* tokens, const int32_t* qo_indptr,
                                const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                int32_t* targets, int32_t* accept, int32_t* emitted,
                                int32_t* new_kv_len, int32_t* dev_err, hipStream_t s) {
  const dim3 rows(static_cast<uint32_t>(B) * max_qo_len);
  if (logits_dt == SDV_F32)
    hipLaunchKernelGGL(sdv_argmax_kernel<SDV_F32>, rows, dim3(kArgmaxThreads), 0, s,
                       reinterpret_cast<const char*>(logits), vocab, qo_indptr, B, targets);
  else
    hipLaunchKernelGGL(sdv_argmax_kernel<SDV_BF16>, rows, dim3(kArgmaxThreads), 0, s,
                       reinterpret_cast<const char*>(logits), vocab, qo_indptr, B, targets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sdv_accept_kernel, dim3((B + 63) / 64), dim3(64), 0, s, targets, tokens,
                     qo_indptr, kv_len, B, max_qo_len, accept, emitted, new_kv_len, dev_err);
  return hipGetLastError();
}

}  // namespace sdv
