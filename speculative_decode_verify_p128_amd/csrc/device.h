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

// ---- ladder top-k of one verify token, by one wave ----
// 64-bit keys (order-preserving score bits << 32 | ~page): the unsigned maximum picks the
// best score and, among equal scores, the lowest page.

// Maximum of v over the wave, the same in every lane: rotate-and-max inside each
// 16-lane row (DPP row_ror, no LDS traffic), then the four row maxima read into scalar
// registers.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  constexpr int kRowRor = 0x120;   // DPP row_ror:n, n = 1 .. 15
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), kRowRor + 1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), kRowRor + 2, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), kRowRor + 4, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), kRowRor + 8, 0xF, 0xF, false)));
  const uint32_t a = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0)),
                         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16)));
  const uint32_t b = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32)),
                         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48)));
  return max(a, b);
}

// One wave selects the k_eff = min(top_k, n) best of the n scores srow[0 .. n-1] (score
// descending, page ascending on ties) in rank order, and every lane calls emit(k, page)
// with the same values.  Lane l holds pages l + 64 i, i < ITEMS (1 <= n <= 64 * ITEMS),
// and caches its largest key.  Each round takes the wave maximum of the cached keys'
// high (score) words; the lanes holding it are a ballot, and only when several lanes tie
// on the score does a second maximum over their low (page) words pick the lowest page.
// The owning lane retires its key and refreshes its cache.  Returns k_eff.
template <int ITEMS, class Emit>
__device__ __forceinline__ int wave_ladder_topk(const float* srow, int n, int top_k, int lane,
                                                Emit&& emit) {
  uint64_t keys[ITEMS];
  uint64_t best = 0;
  // Every lane loads all its items from an index clamped into [0, n) with no branch, so
  // the loads are in flight together; the keys of pages at or beyond n are zeroed after.
  float sv[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) sv[i] = srow[min(lane + kWave * i, n - 1)];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int p = lane + kWave * i;
    keys[i] = p < n ? (static_cast<uint64_t>(ordered_key(sv[i])) << 32) |
                          static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(p))
                    : 0ull;
    best = keys[i] > best ? keys[i] : best;
  }
  const int k_eff = top_k < n ? top_k : n;
  for (int k = 0; k < k_eff; ++k) {
    const uint32_t hi = static_cast<uint32_t>(best >> 32);
    const uint32_t lo = static_cast<uint32_t>(best);
    const uint32_t mhi = wave_max_u32(hi);
    const bool top = hi == mhi;
    const uint64_t tops = __builtin_amdgcn_ballot_w64(top);
    uint32_t mlo;
    int owner;
    if (__builtin_popcountll(tops) == 1) {
      owner = __builtin_ctzll(tops);
      mlo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), owner));
    } else {
      // Equal scores in several lanes (an empty lane's key is 0, below any real key's
      // low word): the largest low word is the lowest page; keys are unique.
      mlo = wave_max_u32(top ? lo : 0u);
      owner = __builtin_ctzll(__builtin_amdgcn_ballot_w64(top && lo == mlo));
    }
    if (lane == owner) {
      uint64_t nb = 0;
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        keys[i] = keys[i] == best ? 0ull : keys[i];
        nb = keys[i] > nb ? keys[i] : nb;
      }
      best = nb;
    }
    emit(k, static_cast<int>(0xffffffffu - mlo));
  }
  return k_eff;
}

// ---- ladder top-k of one verify token by a bit search (wide tables, large top_k) ----
// The same 64-bit keys, lane l holding pages l + 64 i, i < ITEMS.  Its cost does not grow
// with top_k: the k_eff-th largest key T is found bit by bit from the top (the largest T
// that at least k_eff keys reach), and since the page is part of the key, the keys >= T
// are exactly the selection.

template <int ITEMS>
__device__ __forceinline__ void wave_topk_keys(const float* srow, int n, int lane,
                                               uint64_t (&key)[ITEMS]) {
  float sv[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) sv[i] = srow[min(lane + kWave * i, n - 1)];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int p = lane + kWave * i;
    key[i] = p < n ? (static_cast<uint64_t>(ordered_key(sv[i])) << 32) |
                         static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(p))
                   : 0ull;
  }
}

// A threshold T with exactly k_eff = min(top_k, n) of n <= 4096 keys at or above it (1
// when every key is selected), each count a wave sum of per-lane counts (measured faster
// than counting each comparison's lane mask in scalar registers: 15.9 against 16.5 us for
// 1024 pages, top-64, 128 rows); the page word's high 20 bits are the same in every key
// (pages < 4096) and are set at once.  The search stops at the first candidate that
// exactly k_eff keys reach: keys are unique, so those are the k_eff largest, the same
// selection as the k_eff-th largest key itself gives.  Real-valued scores usually leave a
// gap of thousands of ulps between the k_eff-th and the next key, and the search stops
// after 10-26 of its 44 rounds (about 16 on normal scores over 1024 pages, top-64);
// equal scores across the threshold still take every round.
// Sum of v over the wave, the same in every lane: rotate-and-add inside each 16-lane row
// (DPP row_ror), then the four row sums read into scalar registers.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  constexpr int kRowRor = 0x120;
  v += static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), kRowRor + 1, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), kRowRor + 2, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), kRowRor + 4, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), kRowRor + 8, 0xF, 0xF, false));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0)) +
         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16)) +
         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32)) +
         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
}

template <int ITEMS>
__device__ __forceinline__ uint64_t wave_kth_key(const uint64_t (&key)[ITEMS], int n, int k_eff) {
  auto count_ge = [&](uint64_t c) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) m += key[i] >= c ? 1u : 0u;
    return wave_sum_u32(m);
  };
  if (k_eff >= n) return 1ull;
  const uint32_t want = static_cast<uint32_t>(k_eff);
  uint64_t T = 0;
  for (int bit = 63; bit >= 32; --bit) {
    const uint64_t c = T | (1ull << bit);
    const uint32_t m = count_ge(c);
    if (m >= want) {
      T = c;
      if (m == want) return T;
    }
  }
  T |= 0xfffff000ull;
  for (int bit = 11; bit >= 0; --bit) {
    const uint64_t c = T | (1ull << bit);
    const uint32_t m = count_ge(c);
    if (m >= want) {
      T = c;
      if (m == want) return T;
    }
  }
  return T;
}

// Rank of each selected key: the keys >= T of the lanes below come first, then this
// lane's own in item order.
template <int ITEMS>
__device__ __forceinline__ uint32_t wave_selection_offset(const uint64_t (&key)[ITEMS],
                                                          uint64_t T, int lane) {
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) mine += key[i] >= T ? 1u : 0u;
  uint32_t incl = mine;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
  return incl - mine;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off) {
  const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, kWave));
  const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v >> 32), off, kWave));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// The selection of k_eff <= 64 keys in rank order: lane k returns the rank-k key (0 from
// lane k_eff on).  The keys are gathered through st_hi / st_lo (64 words of LDS each,
// used by this wave alone; a wave's LDS accesses take effect in program order) and
// sorted by a bitonic network of lane shuffles.
template <int ITEMS>
__device__ __forceinline__ uint64_t wave_ranked_selection(const uint64_t (&key)[ITEMS], uint64_t T,
                                                          int lane, int k_eff, uint32_t* st_hi,
                                                          uint32_t* st_lo) {
  uint32_t pos = wave_selection_offset(key, T, lane);
#pragma unroll
  for (int i = 0; i < ITEMS; ++i)
    if (key[i] >= T) {
      st_hi[pos] = static_cast<uint32_t>(key[i] >> 32);
      st_lo[pos] = static_cast<uint32_t>(key[i]);
      ++pos;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint64_t v = lane < k_eff ? (static_cast<uint64_t>(st_hi[lane]) << 32) | st_lo[lane] : 0ull;
  // descending: in a block whose lane bit k is 0 the lower lane of each pair keeps the
  // larger key
  for (int k = 2; k <= kWave; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t o = shfl_xor_u64(v, j);
      const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
      v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
    }
  return v;
}

__device__ __forceinline__ int topk_key_page(uint64_t k) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(k));
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
