// Device-side helpers shared by the kernels: element decoding, ordered keys and
// wavefront (64-lane) reductions for CDNA4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sdv.h"

namespace sdv {

constexpr int kWave = 64;
constexpr int kPage = 128;
constexpr int kSub = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two OCP E4M3FN bytes (byte `hi` selects bytes 2-3 instead of 0-1) -> two floats, by
// the gfx950 converter (checked against the format definition for all 256 codes).
template <bool HI>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, float& a, float& b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  f2 v = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HI);
  a = v[0];
  b = v[1];
}

// Decode 16 bytes of stored elements starting at element 0 of the vector into floats.
// F32: 4 values, BF16: 8 values, FP8: 16 values.
template <int DT>
struct Vec16;

template <>
struct Vec16<SDV_F32> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void decode(const uint4& w, float* out) {
    out[0] = __uint_as_float(w.x);
    out[1] = __uint_as_float(w.y);
    out[2] = __uint_as_float(w.z);
    out[3] = __uint_as_float(w.w);
  }
};

template <>
struct Vec16<SDV_BF16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void decode(const uint4& w, float* out) {
    out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x);
    out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
    out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z);
    out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
  }
};

template <>
struct Vec16<SDV_FP8_E4M3> {
  static constexpr int N = 16;
  __device__ __forceinline__ static void decode(const uint4& w, float* out) {
    fp8x2_to_f32<false>(w.x, out[0], out[1]);  fp8x2_to_f32<true>(w.x, out[2], out[3]);
    fp8x2_to_f32<false>(w.y, out[4], out[5]);  fp8x2_to_f32<true>(w.y, out[6], out[7]);
    fp8x2_to_f32<false>(w.z, out[8], out[9]);  fp8x2_to_f32<true>(w.z, out[10], out[11]);
    fp8x2_to_f32<false>(w.w, out[12], out[13]); fp8x2_to_f32<true>(w.w, out[14], out[15]);
  }
};

template <int DT>
constexpr int elem_bytes() { return DT == SDV_F32 ? 4 : (DT == SDV_BF16 ? 2 : 1); }

// One stored element -> float (slow path helpers).
__device__ __forceinline__ float load_elem(const void* base, int64_t idx, int dt) {
  if (dt == SDV_F32) return reinterpret_cast<const float*>(base)[idx];
  if (dt == SDV_BF16) {
    uint32_t h = reinterpret_cast<const uint16_t*>(base)[idx];
    return __uint_as_float(h << 16);
  }
  uint32_t b = reinterpret_cast<const uint8_t*>(base)[idx];
  float a, c;
  fp8x2_to_f32<false>(b, a, c);
  return a;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ void store_out(void* base, int64_t idx, float v, int dt) {
  if (dt == SDV_F32) reinterpret_cast<float*>(base)[idx] = v;
  else reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16_rne(v);
}

// Monotone map of a float to an unsigned key: a < b  <=>  key(a) < key(b) (no NaN).
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);    // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ void set_err(int32_t* dev_err, int32_t bit) {
  if (dev_err) atomicOr(dev_err, bit);
}

// Per-request validation shared by the kernels.  Returns false (and flags) when the
// request's lengths are inconsistent.
__device__ __forceinline__ bool request_lengths(const int32_t* qo_indptr, const int32_t* kv_len,
                                                int r, int B, int max_qo_len, int64_t kv_cap,
                                                int32_t* dev_err, int& row0, int& qo, int& kv) {
  row0 = qo_indptr[r];
  qo = qo_indptr[r + 1] - row0;
  kv = kv_len[r];
  const int64_t rows_cap = static_cast<int64_t>(B) * max_qo_len;
  if (qo < 1 || qo > max_qo_len || kv < qo || row0 < 0 || row0 + qo > rows_cap) {
    set_err(dev_err, SDV_DEVERR_QO_LEN);
    return false;
  }
  if (kv > kv_cap) {
    set_err(dev_err, SDV_DEVERR_KV_CAPACITY);
    return false;
  }
  return true;
}

}  // namespace sdv
