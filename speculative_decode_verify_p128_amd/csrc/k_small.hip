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

// Split-KV combine: LPU = head_dim / 8 lanes per (query row, query head), each lane
// eight channels.  LSE = log sum_s exp(lse_s), out = sum_s exp(lse_s - LSE) * O_s, in
// ascending s; partials with lse = -inf (no keys) are skipped and never read.  A lane
// loads every split's lse at once (with the batch's row range) and then every split's
// partial, so the call costs two memory round trips, not two per split (up to
// kCombineUnroll splits; more loop).
constexpr int kCombineUnroll = 8;

template <int D>
__global__ void __launch_bounds__(256) sdv_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int32_t num_splits,
    int32_t rows_cap, const int32_t* __restrict__ row_begin_dev,
    const int32_t* __restrict__ row_end_dev, int32_t num_heads, void* __restrict__ out,
    int32_t out_dt, float* __restrict__ lse_out) {
  constexpr int LPU = D / 8;
  const int sub = threadIdx.x % LPU;
  const int64_t unit = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / LPU;
  const int64_t units = static_cast<int64_t>(rows_cap) * num_heads;
  if (unit >= units) return;
  const int64_t row = unit / num_heads;
  const int64_t plane = units;   // rows_cap * num_heads
  const int S = num_splits;
  // The first chunk's log-sum-exps load together with the batch's row range (they lie
  // inside the workspace whatever the row), so the range check adds no round trip.
  float l[kCombineUnroll];
#pragma unroll
  for (int k = 0; k < kCombineUnroll; ++k) l[k] = k < S ? part_lse[k * plane + unit] : -INFINITY;
  if (row_begin_dev && (row < *row_begin_dev || row >= *row_end_dev)) return;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float m = -INFINITY, tot = 0.f;
  for (int s0 = 0; s0 < S; s0 += kCombineUnroll) {
    const int n = min(kCombineUnroll, S - s0);
    if (s0 > 0) {
#pragma unroll
      for (int k = 0; k < kCombineUnroll; ++k)
        l[k] = k < n ? part_lse[(s0 + k) * plane + unit] : -INFINITY;
    }
    float mc = m;
#pragma unroll
    for (int k = 0; k < kCombineUnroll; ++k) mc = fmaxf(mc, l[k]);
    if (mc == -INFINITY) continue;
    if (mc > m) {
      // rescale what earlier chunks of splits accumulated to the new reference
      const float f = m == -INFINITY ? 0.f : __expf(m - mc);
      tot *= f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= f;
      m = mc;
    }
    float4 x[kCombineUnroll][2];
#pragma unroll
    for (int k = 0; k < kCombineUnroll; ++k) {
      if (l[k] != -INFINITY) {
        const float4* src = reinterpret_cast<const float4*>(part_o + ((s0 + k) * plane + unit) * D + sub * 8);
        x[k][0] = src[0];
        x[k][1] = src[1];
      }
    }
#pragma unroll
    for (int k = 0; k < kCombineUnroll; ++k) {
      if (l[k] == -INFINITY) continue;
      const float w = __expf(l[k] - m);
      tot += w;
      acc[0] += w * x[k][0].x; acc[1] += w * x[k][0].y; acc[2] += w * x[k][0].z; acc[3] += w * x[k][0].w;
      acc[4] += w * x[k][1].x; acc[5] += w * x[k][1].y; acc[6] += w * x[k][1].z; acc[7] += w * x[k][1].w;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const int64_t idx = unit * D + sub * 8;
  if (out_dt == SDV_BF16) {
    uint16_t* o16 = reinterpret_cast<uint16_t*>(out) + idx;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = static_cast<uint32_t>(f32_to_bf16_rne(acc[2 * k] * inv)) |
             (static_cast<uint32_t>(f32_to_bf16_rne(acc[2 * k + 1] * inv)) << 16);
    *reinterpret_cast<uint4*>(o16) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* o32 = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + idx);
    o32[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    o32[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
  if (lse_out && sub == 0) lse_out[unit] = (m == -INFINITY) ? -INFINITY : m + __logf(tot);
}

hipError_t launch_combine(const float* part_o, const float* part_lse, int32_t num_splits,
                          int32_t rows_cap, const int32_t* row_begin_dev,
                          const int32_t* row_end_dev, int32_t num_heads, int32_t head_dim,
                          void* out, int32_t out_dt, float* lse_out, hipStream_t s) {
  const int64_t units = static_cast<int64_t>(rows_cap) * num_heads;
  if (units == 0) return hipSuccess;
  const int lpu = head_dim / 8;
  const int64_t blocks = (units * lpu + 255) / 256;
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

// Streaming read of a list of equal units (4, 8 or 16 KiB, unit u at base + u * bytes):
// workgroup g takes units g, g + grid, ...; a unit is 256 threads x 1-4 16-byte loads,
// four units in flight per workgroup.  Units outside [0, max_units) are skipped.
__global__ void __launch_bounds__(256) sdv_read_units_probe_kernel(
    const char* __restrict__ base, const int64_t* __restrict__ units, int64_t n_units,
    int64_t max_units, int32_t unit_bytes, uint32_t* __restrict__ sink) {
  constexpr int kInFlight = 4;
  const int per = unit_bytes / (256 * 16);
  uint32_t acc = 0;
  const int64_t grid = gridDim.x;
  for (int64_t u0 = blockIdx.x; u0 < n_units; u0 += kInFlight * grid) {
    uint4 v[kInFlight][4];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const int64_t i = u0 + k * grid;
      const int64_t u = i < n_units ? units[i] : -1;
      const bool ok = u >= 0 && u < max_units;
      const char* p = base + (ok ? u : 0) * unit_bytes;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[k][j] = ok && j < per ? probe_load(reinterpret_cast<const uint4*>(p) + j * 256 + threadIdx.x)
                                : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kInFlight; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc ^= v[k][j].x ^ v[k][j].y ^ v[k][j].z ^ v[k][j].w;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) atomicXor(sink + blockIdx.x, acc);
}

hipError_t launch_read_units_probe(const void* base, const int64_t* units, int64_t n_units,
                                   int64_t max_units, int32_t unit_bytes, uint32_t* sink,
                                   int32_t blocks, hipStream_t s) {
  if (n_units == 0) return hipSuccess;
  hipLaunchKernelGGL(sdv_read_units_probe_kernel, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const char*>(base), units, n_units, max_units, unit_bytes, sink);
  return hipGetLastError();
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
