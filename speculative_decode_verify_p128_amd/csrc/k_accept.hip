// Greedy acceptance of the draft tokens after the verify step.  Acceptance under greedy
// decoding is what "[None][perf] Default Minimax-m3 to unified draft-target kv manager
// ...", Acceptance and accuracy evidence, measures; the verify batch holds qo_len =
// 1 + draft_len tokens per request ("[TRTLLM-14093][feat] Eagle3 for M3 MSA path + CUDA
// graphs compatibility", MSA verify commit).
//
//   1. sdv_argmax_part_kernel: each verify row's logits are cut into parts of 1024
//      16-byte vectors (16 KiB); one 256-thread workgroup per (row, part) holds its part
//      in registers (four non-temporal loads per thread) and writes the part's largest
//      non-NaN value and the lowest index holding it to the workspace.  Many small
//      workgroups keep the memory system busier than one workgroup per row (measured on
//      256 rows x 131072 bf16 logits: 4096 part workgroups finish well ahead of 256
//      1024-thread row workgroups).
//   2. sdv_accept_kernel: one wave per request merges the parts of each of its rows —
//      the largest value, ties to the earlier part, which holds the lower indices — into
//      the target's greedy token after that row (ties to the lowest index, NaN never
//      selected), then takes the longest prefix of drafts equal to the targets of the
//      rows before them, emits them and the bonus target, and writes the corrected
//      kv_len (kv_len - qo_len + 1 + accepted).
#include <climits>

#include "device.h"
#include "internal.h"

namespace sdv {
namespace {

typedef unsigned int u32x4_acc __attribute__((ext_vector_type(4)));

constexpr int kPartThreads = 256;
constexpr int kPartLoads = 4;                              // 16-byte loads per thread
constexpr int kPartVecs = kPartThreads * kPartLoads;       // 16-byte vectors per part

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

// Two passes over the part, held in registers: its largest value M (fmaxf skips NaN; a
// part of NaN leaves M = -inf), reduced over the workgroup, then the lowest index whose
// logit equals M (none, INT_MAX, when the part holds only NaN).  Workgroups of rows
// past qo_indptr[B] (the logits may hold no more rows than that) return at once.
template <int DT>
__global__ void __launch_bounds__(kPartThreads) sdv_argmax_part_kernel(
    const char* __restrict__ logits, int32_t vocab, int32_t parts,
    const int32_t* __restrict__ qo_indptr, int32_t B, float* __restrict__ part_max,
    int32_t* __restrict__ part_idx) {
  constexpr int EB = DT == SDV_F32 ? 4 : 2;
  constexpr int PER = 16 / EB;                 // elements per 16-byte load
  constexpr int NW = kPartThreads / kWave;
  __shared__ float s_max[NW];
  __shared__ int s_idx[NW];
  const int row = blockIdx.x / parts;
  const int part = blockIdx.x - row * parts;
  const int nvec = vocab / PER;
  const int v_begin = part * kPartVecs;
  const int v_end = min(nvec, v_begin + kPartVecs);
  const u32x4_acc* base =
      reinterpret_cast<const u32x4_acc*>(logits + static_cast<int64_t>(row) * vocab * EB);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (row >= qo_indptr[B]) return;
  u32x4_acc w[kPartLoads];
#pragma unroll
  for (int u = 0; u < kPartLoads; ++u) {
    const int v = v_begin + threadIdx.x + u * kPartThreads;
    w[u] = v < v_end ? __builtin_nontemporal_load(base + v) : u32x4_acc{0u, 0u, 0u, 0u};
  }
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < kPartLoads; ++u) {
    if (v_begin + static_cast<int>(threadIdx.x) + u * kPartThreads >= v_end) continue;
    float x[PER];
    decode16<DT>(w[u], x);
#pragma unroll
    for (int k = 0; k < PER; ++k) m = fmaxf(m, x[k]);
  }
  m = wave_max(m);
  if (lane == 0) s_max[wave] = m;
  __syncthreads();
  m = s_max[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) m = fmaxf(m, s_max[k]);
  int best = INT_MAX;
#pragma unroll
  for (int u = 0; u < kPartLoads; ++u) {
    const int v = v_begin + threadIdx.x + u * kPartThreads;
    if (v >= v_end) continue;
    float x[PER];
    decode16<DT>(w[u], x);
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (x[k] == m && v * PER + k < best) best = v * PER + k;
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) best = min(best, __shfl_xor(best, off, kWave));
  if (lane == 0) s_idx[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    int b = s_idx[0];
#pragma unroll
    for (int k = 1; k < NW; ++k) b = min(b, s_idx[k]);
    part_max[blockIdx.x] = m;
    part_idx[blockIdx.x] = b;
  }
}

// The target after one row from its parts (parts in index order, so a strict > keeps
// the lower index on equal values); -1 when every part held only NaN.
__device__ __forceinline__ int merge_parts(const float* __restrict__ part_max,
                                           const int32_t* __restrict__ part_idx, int64_t row,
                                           int parts) {
  const float* pm = part_max + row * parts;
  const int32_t* pi = part_idx + row * parts;
  float m = -INFINITY;
  int b = INT_MAX;
  constexpr int U = 4;
  for (int p0 = 0; p0 < parts; p0 += U) {
    float x[U];
    int i[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      x[k] = p0 + k < parts ? pm[p0 + k] : -INFINITY;
      i[k] = p0 + k < parts ? pi[p0 + k] : INT_MAX;
    }
#pragma unroll
    for (int k = 0; k < U; ++k)
      if (i[k] != INT_MAX && (b == INT_MAX || x[k] > m)) {
        m = x[k];
        b = i[k];
      }
  }
  return b == INT_MAX ? -1 : b;
}

constexpr int kAcceptThreads = 256;   // four requests per workgroup, one wave each

__global__ void __launch_bounds__(kAcceptThreads) sdv_accept_kernel(
    const float* __restrict__ part_max, const int32_t* __restrict__ part_idx, int32_t parts,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ qo_indptr,
    const int32_t* __restrict__ kv_len, int32_t B, int32_t max_qo_len,
    int32_t* __restrict__ targets, int32_t* __restrict__ accept, int32_t* __restrict__ emitted,
    int32_t* __restrict__ new_kv_len, int32_t* dev_err) {
  const int r = blockIdx.x * (kAcceptThreads / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (r >= B) return;
  const int row0 = qo_indptr[r];
  const int qo = qo_indptr[r + 1] - row0;
  const int kv = kv_len[r];
  const int rows = qo_indptr[B];
  int32_t* em = emitted + static_cast<int64_t>(r) * max_qo_len;
  const bool rows_ok = row0 >= 0 && qo >= 1 && static_cast<int64_t>(row0) + qo <= rows &&
                       static_cast<int64_t>(row0) + qo <= static_cast<int64_t>(B) * max_qo_len;
  if (!rows_ok || qo > max_qo_len || kv < qo) {
    // the rows, when they lie inside the batch, still get their targets
    if (rows_ok)
      for (int t = lane; t < qo; t += kWave)
        targets[row0 + t] = merge_parts(part_max, part_idx, row0 + t, parts);
    if (lane == 0) {
      set_err(dev_err, SDV_DEVERR_QO_LEN);
      accept[r] = -1;
      new_kv_len[r] = kv;
    }
    for (int t = lane; t < max_qo_len; t += kWave) em[t] = -1;
    return;
  }
  // Targets of the request's rows, 64 at a time; the first row t < qo - 1 whose target
  // differs from draft t + 1 ends the accepted prefix (a = qo - 1 when none does).
  int a = qo - 1;
  int tgt_a = 0;
  bool found = false;
  for (int t0 = 0; t0 < qo; t0 += kWave) {
    const int t = t0 + lane;
    int tg = 0;
    bool miss = false;
    if (t < qo) {
      tg = merge_parts(part_max, part_idx, row0 + t, parts);
      targets[row0 + t] = tg;
      miss = t < qo - 1 && tokens[row0 + t + 1] != tg;
    }
    if (!found) {
      const uint64_t mb = __ballot(miss);
      const uint64_t last = __ballot(t == qo - 1);
      if (mb) {
        const int l = __builtin_ctzll(mb);
        a = t0 + l;
        tgt_a = __shfl(tg, l, kWave);
        found = true;
      } else if (last) {
        tgt_a = __shfl(tg, __builtin_ctzll(last), kWave);
        found = true;
      }
    }
  }
  for (int t = lane; t < max_qo_len; t += kWave)
    em[t] = t < a ? tokens[row0 + t + 1] : (t == a ? tgt_a : -1);
  if (lane == 0) {
    accept[r] = a;
    new_kv_len[r] = kv - qo + 1 + a;
  }
}

}  // namespace

int32_t greedy_accept_parts(int32_t vocab, int32_t logits_dt) {
  const int per = logits_dt == SDV_F32 ? 4 : 8;
  return (vocab / per + kPartVecs - 1) / kPartVecs;
}

hipError_t launch_greedy_accept(const void* logits, int32_t logits_dt, int32_t vocab,
                                const int32_t* tokens, const int32_t* qo_indptr,
                                const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                void* workspace, int32_t* targets, int32_t* accept,
                                int32_t* emitted, int32_t* new_kv_len, int32_t* dev_err,
                                hipStream_t s) {
  const int32_t parts = greedy_accept_parts(vocab, logits_dt);
  const int64_t rows_cap = static_cast<int64_t>(B) * max_qo_len;
  float* part_max = reinterpret_cast<float*>(workspace);
  int32_t* part_idx = reinterpret_cast<int32_t*>(part_max + rows_cap * parts);
  const dim3 grid(static_cast<uint32_t>(rows_cap * parts));
  if (logits_dt == SDV_F32)
    hipLaunchKernelGGL(sdv_argmax_part_kernel<SDV_F32>, grid, dim3(kPartThreads), 0, s,
                       reinterpret_cast<const char*>(logits), vocab, parts, qo_indptr, B,
                       part_max, part_idx);
  else
    hipLaunchKernelGGL(sdv_argmax_part_kernel<SDV_BF16>, grid, dim3(kPartThreads), 0, s,
                       reinterpret_cast<const char*>(logits), vocab, parts, qo_indptr, B,
                       part_max, part_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RPW = kAcceptThreads / kWave;
  hipLaunchKernelGGL(sdv_accept_kernel, dim3((B + RPW - 1) / RPW), dim3(kAcceptThreads), 0, s,
                     part_max, part_idx, parts, tokens, qo_indptr, kv_len, B, max_qo_len,
                     targets, accept, emitted, new_kv_len, dev_err);
  return hipGetLastError();
}

}  // namespace sdv
