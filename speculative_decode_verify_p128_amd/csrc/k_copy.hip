// Descriptor-driven byte-range copies: the device side of a KV transfer whose
// descriptors a head-slice mapper produced ("[None][perf] Default Minimax-m3 to unified
// draft-target kv manager ...", Root causes and fixes, item 2: one descriptor per
// (layer, K/V, token group) for grouped head-major pages).  Each workgroup takes
// descriptors in turn and streams one with 16-byte non-temporal loads and stores (the
// bytes are moved once; non-temporal stores measured 132 -> 122 us on the draft layer's
// 645 MB of reads and writes); a descriptor outside its buffers or off the 16-byte grid
// is skipped and flagged.
#include "device.h"
#include "internal.h"

namespace sdv {
namespace {

typedef unsigned int u32x4_copy __attribute__((ext_vector_type(4)));
constexpr int kCopyUnroll = 4;

__global__ void __launch_bounds__(256) sdv_copy_desc_kernel(
    const char* __restrict__ src, int64_t src_bytes, char* __restrict__ dst, int64_t dst_bytes,
    const sdv_copy_desc* __restrict__ descs, int32_t n, int32_t* dev_err) {
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const sdv_copy_desc e = descs[i];
    const bool ok = e.bytes >= 0 && e.src_offset >= 0 && e.dst_offset >= 0 &&
                    ((e.src_offset | e.dst_offset | e.bytes) & 15) == 0 &&
                    e.bytes <= src_bytes - e.src_offset && e.bytes <= dst_bytes - e.dst_offset;
    if (!ok) {
      if (threadIdx.x == 0) set_err(dev_err, SDV_DEVERR_COPY_RANGE);
      continue;
    }
    const u32x4_copy* s = reinterpret_cast<const u32x4_copy*>(src + e.src_offset);
    u32x4_copy* d = reinterpret_cast<u32x4_copy*>(dst + e.dst_offset);
    const int64_t n16 = e.bytes / 16;
    // kCopyUnroll loads in flight per thread before the stores (a 16 KiB descriptor in
    // one round)
    for (int64_t k0 = threadIdx.x; k0 < n16; k0 += kCopyUnroll * blockDim.x) {
      u32x4_copy v[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t k = k0 + static_cast<int64_t>(u) * blockDim.x;
        if (k < n16) v[u] = __builtin_nontemporal_load(s + k);
      }
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t k = k0 + static_cast<int64_t>(u) * blockDim.x;
        if (k < n16) __builtin_nontemporal_store(v[u], d + k);
      }
    }
  }
}

}  // namespace

hipError_t launch_copy_descriptors(const void* src, size_t src_bytes, void* dst, size_t dst_bytes,
                                  const sdv_copy_desc* descs, int32_t n, int32_t* dev_err,
                                  hipStream_t s) {
  const int blocks = n < 8192 ? n : 8192;
  hipLaunchKernelGGL(sdv_copy_desc_kernel, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const char*>(src), static_cast<int64_t>(src_bytes),
                     reinterpret_cast<char*>(dst), static_cast<int64_t>(dst_bytes), descs, n,
                     dev_err);
  return hipGetLastError();
}

}  // namespace sdv
