// Greedy acceptance of the draft tokens after the verify step.  Acceptance under greedy
// decoding is what "[None][perf] Default Minimax-m3 to unified draft-target kv manager
// ...", Acceptance and accuracy evidence, measures; the verify batch holds qo_len =
// 1 + draft_len tokens per request ("[TRTLLM-14093][feat] Eagle3 for M3 MSA path + CUDA
// graphs compatibility", MSA verify commit).
//
//   1. sdv_argmax_part_kernel: each verify row's logits are cut into parts of 1024
//      16-byte vectors (16 KiB); one 256-thread workgroup per (row, part) holds its part
//      in registers (four non-temporal loads per thread) and writes the part's largest
//      non-NaN value and the lowest index holding it to the workspace, as one 64-bit key:
//      the order-preserving bits of the value above the complemented index, so that the
//      largest key is the largest value at the lowest index (0: a part of NaN only).
//      Many small workgroups keep the memory system busier than one workgroup per row
//      (measured on 256 rows x 131072 bf16 logits: 4096 part workgroups finish well
//      ahead of 256 1024-thread row workgroups).
//   2. sdv_accept_kernel: one wave per request takes the largest key of each of its rows
//      — the target's greedy token after that row (ties to the lowest index, NaN never
//      selected) — with its lanes spread over (row, part) pairs, so that every key and
//      draft token is loaded in one round; then it takes the longest prefix of drafts
//      equal to the targets of the rows before them, emits them and the bonus target,
//      and writes the corrected kv_len (kv_len - qo_len + 1 + accepted).  The kernel is a
//      chain of dependent loads (lengths, keys, outputs), so loads issued together are
//      what its time depends on.
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
    const int32_t* __restrict__ qo_indptr, int32_t B, uint64_t* __restrict__ part_keys) {
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
    part_keys[blockIdx.x] = b == INT_MAX ? 0ull
                                         : (static_cast<uint64_t>(ordered_key(m)) << 32) |
                                               static_cast<uint32_t>(~static_cast<uint32_t>(b));
  }
}

__device__ __forceinline__ int key_target(uint64_t k) {
  return k == 0 ? -1 : static_cast<int>(~static_cast<uint32_t>(k));
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off) {
  const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, kWave));
  const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v >> 32), off, kWave));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

constexpr int kAcceptThreads = 256;   // four requests per workgroup, one wave each

// pshift: log2 of the lane segment that holds one row's parts (parts <= 64), or -1 when
// a row has more than 64 parts (then rows are merged one after another).
__global__ void __launch_bounds__(kAcceptThreads) sdv_accept_kernel(
    const uint64_t* __restrict__ part_keys, int32_t parts, int32_t pshift,
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
  const bool usable = rows_ok && qo <= max_qo_len && kv >= qo;
  // Targets of the request's rows (also when its other lengths are unusable, as long as
  // its rows lie inside the batch); the first row t < qo - 1 whose target differs from
  // draft t + 1 ends the accepted prefix (a = qo - 1 when none does).
  int a = qo - 1;
  int tgt_a = 0;
  bool found = !usable;
  if (rows_ok && pshift >= 0) {
    const int seg = 1 << pshift;           // lanes per row, >= parts
    const int rpp = kWave >> pshift;       // rows per pass
    const int sub = lane >> pshift;
    const int p = lane & (seg - 1);
    for (int t0 = 0; t0 < qo; t0 += rpp) {
      const int t = t0 + sub;
      uint64_t k = 0;
      int draft = 0;
      if (t < qo && p < parts) k = part_keys[(static_cast<int64_t>(row0) + t) * parts + p];
      if (p == 0 && t < qo - 1) draft = tokens[row0 + t + 1];
      for (int off = seg >> 1; off >= 1; off >>= 1) k = max_u64(k, shfl_xor_u64(k, off));
      const int tg = key_target(k);
      const bool lead = p == 0 && t < qo;
      if (lead) targets[row0 + t] = tg;
      if (!found) {
        const uint64_t mb = __ballot(lead && t < qo - 1 && draft != tg);
        const uint64_t last = __ballot(lead && t == qo - 1);
        if (mb) {
          const int l = __builtin_ctzll(mb);
          a = t0 + (l >> pshift);
          tgt_a = __shfl(tg, l, kWave);
          found = true;
        } else if (last) {
          tgt_a = __shfl(tg, __builtin_ctzll(last), kWave);
          found = true;
        }
      }
    }
  } else if (rows_ok) {
    for (int t = 0; t < qo; ++t) {
      const uint64_t* pk = part_keys + (static_cast<int64_t>(row0) + t) * parts;
      uint64_t k = 0;
      for (int p = lane; p < parts; p += kWave) k = max_u64(k, pk[p]);
      for (int off = kWave >> 1; off >= 1; off >>= 1) k = max_u64(k, shfl_xor_u64(k, off));
      const int tg = key_target(k);
      if (lane == 0) targets[row0 + t] = tg;
      if (!found && (t == qo - 1 || tokens[row0 + t + 1] != tg)) {
        a = t;
        tgt_a = tg;
        found = true;
      }
    }
  }
  if (!usable) {
    if (lane == 0) {
      set_err(dev_err, SDV_DEVERR_QO_LEN);
      accept[r] = -1;
      new_kv_len[r] = kv;
    }
    for (int t = lane; t < max_qo_len; t += kWave) em[t] = -1;
    return;
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
  uint64_t* part_keys = reinterpret_cast<uint64_t*>(workspace);
  int32_t pshift = -1;
  if (parts <= kWave) {
    pshift = 0;
    while ((1 << pshift) < parts) ++pshift;
  }
  const dim3 grid(static_cast<uint32_t>(rows_cap * parts));
  if (logits_dt == SDV_F32)
    hipLaunchKernelGGL(sdv_argmax_part_kernel<SDV_F32>, grid, dim3(kPartThreads), 0, s,
                       reinterpret_cast<const char*>(logits), vocab, parts, qo_indptr, B,
                       part_keys);
  else
    hipLaunchKernelGGL(sdv_argmax_part_kernel<SDV_BF16>, grid, dim3(kPartThreads), 0, s,
                       reinterpret_cast<const char*>(logits), vocab, parts, qo_indptr, B,
                       part_keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RPW = kAcceptThreads / kWave;
  hipLaunchKernelGGL(sdv_accept_kernel, dim3((B + RPW - 1) / RPW), dim3(kAcceptThreads), 0, s,
                     part_keys, parts, pshift, tokens, qo_indptr, kv_len, B, max_qo_len,
                     targets, accept, emitted, new_kv_len, dev_err);
  return hipGetLastError();
}

}  // namespace sdv
