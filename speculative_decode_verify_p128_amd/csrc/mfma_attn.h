// Device helpers shared by the matrix-core verify-attention kernels (gfx950, wave64,
// v_mfma_f32_16x16x32_bf16): operand layouts, LDS block geometry, explicit waits.
//
// Score tiles are computed transposed, S^T = K Q^T, with K the A operand (lane l: token
// l % 16, 8 channels of a 32-channel step) and Q^T the B operand; the result leaves lane
// l holding query row l % 16 for tokens 4(l/16) .. +3 of each 16-token tile, which is
// the B operand of O^T = V^T P^T.  Channels inside a 32-channel step are permuted the
// same way for K and Q (lane group q takes channels q*d/4 .. q*d/4 + d/4 - 1 across the
// steps), which leaves the dot products unchanged.  K/V blocks of 32 tokens sit in LDS
// with their 16-byte chunks XOR-swizzled by row, so the operand reads (16 rows, one
// column) and the value reads (one row) are free of bank conflicts.
#pragma once

#include <type_traits>

#include "device.h"
#include "internal.h"

namespace sdv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kRescaleLog2 = 8.f;

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Workgroup barrier for the block ring without a memory fence.  __syncthreads() also
// releases all of the wave's outstanding memory operations, which would drain every
// asynchronous copy in flight; here the waits are explicit (vmcnt for the copies of the
// block about to be read, lgkmcnt for the reads of a slot about to be refilled) and
// only the compiler is kept from moving LDS accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Geometry of one 32-token block of one head in LDS.
template <int D, int KDT>
struct Geo {
  static constexpr int EB = elem_bytes<KDT>();
  static constexpr int ROWB = D * EB;               // bytes per token row
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;              // rows per wave load instruction
  static constexpr int HALF = 32 * ROWB;            // K (or V) bytes of one block
  static constexpr int BLOCK = 2 * HALF;            // K then V
  static constexpr int LPT = (2 * 32 / RPI) / 4;    // load instructions per wave per block
  static constexpr int STEPS = D / 32;              // 32-channel MFMA steps
  static constexpr int NT = D / 16;                 // 16-channel output tiles
  static_assert(LPT >= 1, "block too small for four waves");
  // byte offset in a block's K or V half of (row, byte-in-row)
  __device__ static __forceinline__ int at(int row, int byte) {
    const int chunk = byte >> 4;
    return row * ROWB + (((chunk ^ row) & (CPR - 1)) << 4) + (byte & 15);
  }
};

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}

template <int NB>
__device__ __forceinline__ void lds_read(const char* p, uint32_t* w) {
  if constexpr (NB == 16) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (NB == 8) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x; w[1] = x.y;
  } else if constexpr (NB == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (NB == 2) {
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else {
    w[0] = *reinterpret_cast<const uint8_t*>(p);
  }
}

// Token of the 32-token block that element e (0..7) of lane group q stands for in the
// value product: the score tile of tokens 0-15 gives e < 4, the one of 16-31 e >= 4.
__device__ __forceinline__ int ptok(int q, int e) { return e < 4 ? 4 * q + e : 12 + 4 * q + e; }

template <int D, int KDT>
__device__ __forceinline__ bf16x8 k_operand(const char* kb, int tt, int s, int i, int q) {
  using Gm = Geo<D, KDT>;
  const int row = tt * 16 + i;
  const int byte = (q * (D / 4) + s * 8) * Gm::EB;
  uint32_t w[4];
  if constexpr (KDT == SDV_BF16) {
    lds_read<16>(kb + Gm::at(row, byte), w);
  } else {
    uint32_t r8[2];
    lds_read<8>(kb + Gm::at(row, byte), r8);
    float f[8];
    fp8x2_to_f32<false>(r8[0], f[0], f[1]);
    fp8x2_to_f32<true>(r8[0], f[2], f[3]);
    fp8x2_to_f32<false>(r8[1], f[4], f[5]);
    fp8x2_to_f32<true>(r8[1], f[6], f[7]);
    w[0] = pack2_bf16(f[0], f[1]);
    w[1] = pack2_bf16(f[2], f[3]);
    w[2] = pack2_bf16(f[4], f[5]);
    w[3] = pack2_bf16(f[6], f[7]);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// A operands of O^T += V^T P^T for this wave's output tiles n0 .. n0 + NTW - 1: element
// e of tile n is V[ptok(q, e)][NT * i + n0 + n].  v_runs reads, for each of the lane's 8
// tokens, its run of NTW channels; v_zero_tail clears the runs of positions past kv_len;
// v_operand interleaves bf16 runs into an operand with byte permutes, or widens fp8 runs
// exactly to bf16.
template <int D, int KDT, int NTW>
__device__ __forceinline__ void v_runs(const char* vb, int i, int q, int n0,
                                       uint32_t (&raw)[8][4]) {
  using Gm = Geo<D, KDT>;
  constexpr int NBYTES = NTW * Gm::EB;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int tok = ptok(q, e);
    const int byte = (Gm::NT * i + n0) * Gm::EB;
    raw[e][0] = raw[e][1] = raw[e][2] = raw[e][3] = 0u;
    lds_read<NBYTES>(vb + Gm::at(tok, byte), raw[e]);
  }
}

__device__ __forceinline__ void v_zero_tail(int q, int pos0, int kv, uint32_t (&raw)[8][4]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (pos0 + ptok(q, e) >= kv) raw[e][0] = raw[e][1] = raw[e][2] = raw[e][3] = 0u;
}

template <int KDT>
__device__ __forceinline__ bf16x8 v_operand(const uint32_t (&raw)[8][4], int n) {
  uint32_t w[4];
  if constexpr (KDT == SDV_BF16) {
    const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      w[m] = __builtin_amdgcn_perm(raw[2 * m + 1][n >> 1], raw[2 * m][n >> 1], sel);
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float a0, a1, b0, b1;
      const uint32_t wa = raw[2 * m][n >> 2];
      const uint32_t wb = raw[2 * m + 1][n >> 2];
      if ((n & 2) == 0) {
        fp8x2_to_f32<false>(wa, a0, a1);
        fp8x2_to_f32<false>(wb, b0, b1);
      } else {
        fp8x2_to_f32<true>(wa, a0, a1);
        fp8x2_to_f32<true>(wb, b0, b1);
      }
      w[m] = (n & 1) ? pack2_bf16(a1, b1) : pack2_bf16(a0, b0);
    }
  }
  return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

constexpr int kMaxDenseBlocks = 1024;   // 32-token blocks per dense split

// f(integral_constant<int, I>) for I = 0 .. N - 1, unrolled at compile time.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Waits until at most `after` blocks' copies (LPT instructions each) of this wave are
// still in flight, for after in [0, MAXA].
template <int LPT, int MAXA>
__device__ __forceinline__ void wait_blocks(int after) {
  if constexpr (MAXA > 0) {
    if (after >= MAXA) {
      wait_vmcnt<MAXA * LPT>();
      return;
    }
    wait_blocks<LPT, MAXA - 1>(after);
  } else {
    wait_vmcnt<0>();
  }
}

// Blocks per dense split for this launch.  One length for all workgroups, so that they
// get equal numbers of blocks whatever the mix of request lengths: about the launch's
// total blocks over all (request, KV head) pairs divided by the workgroups the GPU holds
// at once, at least what num_splits splits need for the longest request, and at most
// the 1024 blocks whose metadata a workgroup stages (the caller guarantees that
// ceil(max_sub_pages / num_splits) fits).  All threads call; wave 0 reads every kv_len.
__device__ inline int dense_chunk(const AttnArgs& a, const DenseSource& ds, int* slot_lds) {
  const int tid = threadIdx.x;
  if (tid < kWave) {
    int64_t sum = 0;
    int mx = 0;
    for (int rr = tid; rr < a.B; rr += kWave) {
      const int64_t k = a.kv_len[rr];
      const int nb = static_cast<int>(k <= 0 ? 0 : min<int64_t>((k + kSub - 1) / kSub, ds.max_sub_pages));
      sum += nb;
      mx = max(mx, nb);
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
      sum += __shfl_xor(sum, off, kWave);
      mx = max(mx, __shfl_xor(mx, off, kWave));
    }
    if (tid == 0) {
      // Rounding each pair's chunk count up adds about half a chunk per pair, so aim the
      // total at the resident count less half a workgroup per pair (at least half of it).
      const int64_t pairs = static_cast<int64_t>(a.B) * a.num_kv_heads;
      const int64_t full = a.target_wgs > 0 ? a.target_wgs : 1;
      const int64_t tgt = max<int64_t>(full - pairs / 2, (full + 1) / 2);
      int64_t c = (sum * a.num_kv_heads + tgt - 1) / tgt;
      c = max<int64_t>(c, (mx + a.num_splits - 1) / a.num_splits);
      c = min<int64_t>(c, kMaxDenseBlocks);
      *slot_lds = static_cast<int>(max<int64_t>(c, 1));
    }
  }
  __syncthreads();
  return *slot_lds;
}

struct NoUnion {};

// P32 page index of the K sub-page of a dense split's blocks; -1 marks an index outside
// the pool.  The view's geometry puts V one P128 page (four P32 pages) after K.
struct DenseMeta {
  int32_t xk[kMaxDenseBlocks];
};

}  // namespace
}  // namespace sdv
