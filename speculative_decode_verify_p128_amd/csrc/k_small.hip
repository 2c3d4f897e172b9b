// Small kernels: P32 sub-page offsets of the draft view, split-KV combine, fill.
#include "device.h"
#include "internal.h"

namespace sdv {

// One thread per (request, 32-token sub-page of the block-table capacity).
// Sub-page i of request r lies in P128 slot block_table[r][i / 4], token group i % 4;
// counted in P32 pages from the view root, its K page is 4 * stride * slot + i % 4 and
// its V page four P32 pages (one P128 page) further.  ("[None][perf] wrap up eagle
// changes in m3 side branch", draft-view index-scale commit; "[None][perf] Default
// Minimax-m3 to unified draft-target kv manager ...", item 2 Grouped-HND.)
__global__ void __launch_bounds__(256) sdv_subpage_offsets_kernel(
    const int32_t* __restrict__ block_table, int32_t B, int32_t max_blocks, int32_t bt_stride,
    int32_t slot_stride, int32_t num_slots, int32_t* __restrict__ sub_offsets,
    int32_t* dev_err) {
  const int64_t per = 4ll * max_blocks;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= per * B) return;
  const int64_t r = i / per;
  const int32_t sp = static_cast<int32_t>(i - r * per);
  int32_t slot = block_table[r * bt_stride + (sp >> 2)];
  if (slot < 0 || slot >= num_slots) {
    set_err(dev_err, SDV_DEVERR_PAGE_RANGE);
    slot = 0;
  }
  const int32_t k_idx = slot * slot_stride * 4 + (sp & 3);
  sub_offsets[(r * 2 + 0) * per + sp] = k_idx;
  sub_offsets[(r * 2 + 1) * per + sp] = k_idx + 4;
}

hipError_t launch_subpage_offsets(const int32_t* block_table, int32_t B, int32_t max_blocks,
                                  int32_t bt_stride, int32_t slot_stride, int32_t num_slots,
                                  int32_t* sub_offsets, int32_t* dev_err, hipStream_t s) {
  const int64_t n = 4ll * max_blocks * B;
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(sdv_subpage_offsets_kernel, dim3(static_cast<uint32_t>(blocks)),
                     dim3(threads), 0, s, block_table, B, max_blocks, bt_stride, slot_stride,
                     num_slots, sub_offsets, dev_err);
  return hipGetLastError();
}

// Split-KV combine: one wave per (query row, query head); each lane owns head_dim / 64
// channels.  LSE = log sum_s exp(lse_s), out = sum_s exp(lse_s - LSE) * O_s; partials
// with lse = -inf (no keys) are skipped and never read.
template <int D>
__global__ void __launch_bounds__(256) sdv_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int32_t num_splits,
    int32_t rows_cap, const int32_t* __restrict__ row_begin_dev,
    const int32_t* __restrict__ row_end_dev, int32_t num_heads, void* __restrict__ out,
    int32_t out_dt, float* __restrict__ lse_out) {
  constexpr int PER = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t units = static_cast<int64_t>(rows_cap) * num_heads;
  if (unit >= units) return;
  const int64_t row = unit / num_heads;
  if (row_begin_dev && (row < *row_begin_dev || row >= *row_end_dev)) return;
  const int64_t plane = units;   // rows_cap * num_heads
  float m = -INFINITY;
  for (int s = 0; s < num_splits; ++s) m = fmaxf(m, part_lse[s * plane + unit]);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < num_splits; ++s) {
      const float l = part_lse[s * plane + unit];
      if (l == -INFINITY) continue;
      const float w = __expf(l - m);
      tot += w;
      const float* src = part_o + (s * plane + unit) * D;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += w * src[lane * PER + e];
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) store_out(out, unit * D + lane * PER + e, acc[e] * inv, out_dt);
  if (lse_out && lane == 0) lse_out[unit] = (m == -INFINITY) ? -INFINITY : m + __logf(tot);
}

hipError_t launch_combine(const float* part_o, const float* part_lse, int32_t num_splits,
                          int32_t rows_cap, const int32_t* row_begin_dev,
                          const int32_t* row_end_dev, int32_t num_heads, int32_t head_dim,
                          void* out, int32_t out_dt, float* lse_out, hipStream_t s) {
  const int64_t units = static_cast<int64_t>(rows_cap) * num_heads;
  if (units == 0) return hipSuccess;
  const int waves_per_block = 4;
  const int64_t blocks = (units + waves_per_block - 1) / waves_per_block;
  if (head_dim == 128)
    hipLaunchKernelGGL(sdv_combine_kernel<128>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                       part_o, part_lse, num_splits, rows_cap, row_begin_dev, row_end_dev, num_heads, out,
                       out_dt, lse_out);
  else
    hipLaunchKernelGGL(sdv_combine_kernel<64>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                       part_o, part_lse, num_splits, rows_cap, row_begin_dev, row_end_dev, num_heads, out,
                       out_dt, lse_out);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) sdv_fill_kernel(uint4* __restrict__ dst, int64_t n16,
                                                       uint32_t pattern) {
  const uint4 v = make_uint4(pattern, pattern, pattern, pattern);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    dst[i] = v;
}

typedef unsigned int u32x4_probe __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 probe_load(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_probe*>(p)));
}

// Streaming-read probe: every byte of src read once with non-temporal 16-byte loads (4
// in flight per lane), folded into one word per workgroup so the loads cannot be elided.
__global__ void __launch_bounds__(256) sdv_read_probe_kernel(const uint4* __restrict__ src,
                                                             int64_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = probe_load(src + i), b = probe_load(src + i + stride),
                c = probe_load(src + i + 2 * stride), d = probe_load(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = probe_load(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) atomicXor(sink + blockIdx.x, acc);
}

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                             hipStream_t s) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(sdv_read_probe_kernel, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(src), n16, sink);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* dst, size_t bytes, uint32_t pattern, hipStream_t s) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(sdv_fill_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(dst), n16, pattern);
  return hipGetLastError();
}

}  // namespace sdv
