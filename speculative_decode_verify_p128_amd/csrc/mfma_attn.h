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
#include "sparse_union.h"

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

// Two OCP E4M3FN bytes (the low half of w, or the high half) widened to two bf16 in one
// instruction (v_cvt_scalef32_pk_bf16_fp8 with scale 1): exact, since every E4M3FN value
// is a bf16 value.  The first byte lands in the low half.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
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

// LDS banking of 16-byte reads on gfx950 (measured with exec-masked probes under
// SQ_LDS_BANK_CONFLICT): a wave's ds_read_b128 is served in four passes of 16 lanes —
// lanes with the same lane bit 5 and the same parity of lane bits 2, 3 and 4 — and a
// pass is conflict-free when its 16 lanes hit 16 different 16-byte bank groups
// (address / 16 mod 16, 64 banks).  The operand reads put lane (i = l % 16, q = l / 16)
// on row i (K) or on a row fixed by q (V), with the 16-byte chunk fixed by q or by i;
// XOR-ing chunks with a key of the row whose bits 2 and 3 are equal keeps the two lane
// quarters of every pass in opposite parity classes of bank groups, so both read
// patterns are conflict-free (a plain XOR with row % 16 leaves them 2-way conflicting).
__device__ __forceinline__ constexpr int row_key16(int row) {
  return (row & 7) | ((row & 4) << 1);
}

// Geometry of one 32-token block of one head in LDS.
//
// fp8 rows of 128 channels (128 bytes, eight 16-byte chunks) are read 8 bytes a lane
// (ds_read_b64), which gfx950 serves in two passes, lanes 0-31 and 32-63 (measured with
// lane-pair probes under SQ_LDS_BANK_CONFLICT); a pass is conflict-free when its 32 lanes
// hit 32 different 8-byte bank pairs.  With the 16-byte layout's row-only XOR, the K
// operand reads (rows i = 0..15 of lane groups q, one 8-byte half of a chunk) met 4-way
// conflicts and the value reads (four token rows, one per lane group) 2-way.  For this
// shape the layout also swaps rows 4-7 of every eight in pairs (prow), XORs chunks with
// row / 2, and the lane groups take their four 8-channel units of a step in the order
// s ^ (q & 1) (step_unit), so that the two lane groups of a pass read opposite halves of
// their chunks: both read patterns measured conflict-free.
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
  static constexpr bool B64_ROWS = KDT == SDV_FP8_E4M3 && D == 128;   // the 8-byte-read layout
  static_assert(LPT >= 1, "block too small for four waves");
  // LDS row of token row `row` inside its group of eight (an involution)
  __device__ static __forceinline__ constexpr int prow(int row) {
    return B64_ROWS ? row ^ ((row >> 2) & 1) : row;
  }
  // XOR key of a row's 16-byte chunks (rows of 16 chunks: row_key16; rows of 8 chunks
  // start every other row in the other half of the bank groups by themselves)
  __device__ static __forceinline__ constexpr int swz(int row) {
    return B64_ROWS ? (row >> 1) & 7 : (CPR == 16 ? row_key16(row) : row & (CPR - 1));
  }
  // byte offset in a block's K or V half of (row, byte-in-row)
  __device__ static __forceinline__ int at(int row, int byte) {
    const int chunk = byte >> 4;
    return prow(row) * ROWB + (((chunk ^ swz(row)) & (CPR - 1)) << 4) + (byte & 15);
  }
  // byte offset in the global K or V run of the chunk that lands at LDS position
  // (lds_row, lds_chunk): the inverse of at()
  __device__ static __forceinline__ int src(int lds_row, int lds_chunk) {
    const int row = prow(lds_row);
    return row * ROWB + (((lds_chunk ^ swz(row)) & (CPR - 1)) << 4);
  }
  // 8-channel unit of its quarter row that lane group q feeds the matrix core at step s
  // (the same for K and for Q, so the dot products are unchanged)
  __device__ static __forceinline__ constexpr int step_unit(int q, int s) {
    return B64_ROWS ? s ^ (q & 1) : s;
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
  const int byte = (q * (D / 4) + Gm::step_unit(q, s) * 8) * Gm::EB;
  uint32_t w[4];
  if constexpr (KDT == SDV_BF16) {
    lds_read<16>(kb + Gm::at(row, byte), w);
  } else {
    uint32_t r8[2];
    lds_read<8>(kb + Gm::at(row, byte), r8);
    w[0] = fp8x2_to_bf16x2<false>(r8[0]);
    w[1] = fp8x2_to_bf16x2<true>(r8[0]);
    w[2] = fp8x2_to_bf16x2<false>(r8[1]);
    w[3] = fp8x2_to_bf16x2<true>(r8[1]);
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
    // byte (n & 3) of wa and of wb side by side in the low half of one word, widened
    // together (one byte permute and one conversion per output word)
    const uint32_t sel = 0x0c0c0400u + (n & 3) * 0x0101u;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t wa = raw[2 * m][n >> 2];
      const uint32_t wb = raw[2 * m + 1][n >> 2];
      w[m] = fp8x2_to_bf16x2<false>(__builtin_amdgcn_perm(wb, wa, sel));
    }
  }
  return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// A wave's share of one block copy: LPT asynchronous 16-byte-per-lane loads that
// together copy one block (K then V) into a ring slot; lane l of instruction n lands at
// slot + (n * 64 + l) * 16.  The per-lane source offsets inside the block's K or V run
// and the LDS offsets inside the slot do not change from block to block, so a copy is
// a scalar block base, a constant 32-bit lane offset and M0.
template <int D, int KDT>
struct BlockCopier {
  using Gm = Geo<D, KDT>;
  uint32_t off[Gm::LPT];      // lane's byte offset in the K or V run of the block
  uint32_t lds[Gm::LPT];      // LDS byte offset of the instruction in the slot (uniform)
  bool is_v[Gm::LPT];         // copies V rather than K (uniform)

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int n = 0; n < Gm::LPT; ++n) {
      const int ins = wave * Gm::LPT + n;               // 0 .. 2 * 32 / RPI - 1
      const int half = ins / (32 / Gm::RPI);            // 0 = K, 1 = V
      const int row = (ins % (32 / Gm::RPI)) * Gm::RPI + lane / Gm::CPR;
      off[n] = static_cast<uint32_t>(Gm::src(row, lane % Gm::CPR));
      lds[n] = static_cast<uint32_t>(half * Gm::HALF + (ins % (32 / Gm::RPI)) * 64 * 16);
      is_v[n] = half != 0;
    }
  }

  // kbase, vbase: first byte of the block's K and V runs; slot_lds: LDS address of the
  // ring slot.  All three are wave-uniform.
  __device__ __forceinline__ void issue(uint64_t kbase, uint64_t vbase, uint32_t slot_lds) const {
#pragma unroll
    for (int n = 0; n < Gm::LPT; ++n) {
      const uint64_t base = is_v[n] ? vbase : kbase;
      const uint32_t m0 = slot_lds + lds[n];
      // Inline assembly, so that the compiler's wait insertion, which cannot tell ring
      // slots apart, does not drain the copies in flight before every LDS read; the
      // ring's own vmcnt waits and barriers order copies and reads.  M0 (the copy's
      // LDS base) is reserved by the compiler, which uses it in this kernel for
      // nothing else; the clobber records that it is overwritten.  The copies are
      // non-temporal: every K/V byte is read once.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                   :
                   : "s"(m0), "v"(off[n]), "s"(base)
                   : "memory", "m0");
#pragma clang diagnostic pop
    }
  }
};

constexpr int kMaxDenseBlocks = kMaxSplitBlocks;   // 32-token blocks per dense split

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
__device__ inline int dense_chunk(const AttnArgs& a, int max_blocks, int* slot_lds) {
  const int tid = threadIdx.x;
  if (tid < kWave) {
    int64_t sum = 0;
    int mx = 0;
    for (int rr = tid; rr < a.B; rr += kWave) {
      const int64_t k = a.kv_len[rr];
      const int nb = static_cast<int>(k <= 0 ? 0 : min<int64_t>((k + kSub - 1) / kSub, max_blocks));
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

// Dense split-KV pieces sized to the requests (ring kernel, num_splits > 1).  Each
// (request, KV head) pair with nb blocks is cut into k = max(1, ceil(nb / c)) near-equal
// runs, c the smallest run length for which all pairs' runs fit the workgroups the GPU
// holds at once and no pair needs more than num_splits of them (its partial slots), so
// that every workgroup with work is resident from the start and none carries more than
// c blocks; one run length for all pairs instead puts up to num_splits runs of the
// longest request's length on a CU while short requests leave theirs idle.  The runs
// are numbered level by level (every pair's run 0, then run 1 of the pairs with two or
// more, ...), pairs in request-major order, and grid position lin (dispatch order) takes
// run lin; positions past the last run return false.  B <= kCompactMaxRequests.  All
// threads call; wave 0 reads every request's lengths (one round trip); lds holds 9 ints.
constexpr int kCompactMaxRequests = 512;

struct DensePiece {
  int r, h, j;       // request, KV head, run (= partial slot)
  int first, n;      // blocks [first, first + n) of the request
  int k;             // runs of the pair
  int row0, qo, kv;  // the request's first query row, query rows and KV length
};

// ceil(v / c) for 0 <= v <= 2^20, c >= 1, rc within a few ulp of 1 / c: the float
// quotient is then within 1 of v / c and one correction step makes it exact (an integer
// division is a long instruction sequence, and the search below takes many)
__device__ __forceinline__ int ceil_div_small(int v, int c, float rc) {
  int q = static_cast<int>(static_cast<float>(v) * rc);
  q += (q + 1) * c <= v ? 1 : 0;
  q -= q * c > v ? 1 : 0;
  return q + (q * c < v ? 1 : 0);
}

// NI: request slots a lane of wave 0 holds (B <= 64 * NI).
template <int NI>
__device__ inline bool dense_compact_piece_t(const AttnArgs& a, int max_blocks, int* lds,
                                             DensePiece& pc) {
  const int tid = threadIdx.x;
  const int Hkv = a.num_kv_heads;
  const int S = a.num_splits;
  const int lin = static_cast<int>(blockIdx.y * gridDim.x + blockIdx.x);
  if (tid < kWave) {
    const int lane = tid;
    const int ni = (a.B + kWave - 1) / kWave;   // item slots in use (wave-uniform)
    int nb[NI], row0s[NI], qos[NI], kvs[NI];
    int sum = 0, mx = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rr = lane + kWave * i;
      int v = 0, r0 = 0, q1 = 0, kk = 0;
      if (i < ni && rr < a.B) {
        kk = a.kv_len[rr];
        r0 = a.qo_indptr[rr];
        q1 = a.qo_indptr[rr + 1];
        v = kk <= 0 ? 0 : min((kk + kSub - 1) / kSub, max_blocks);
      }
      nb[i] = v;
      row0s[i] = r0;
      qos[i] = q1 - r0;
      kvs[i] = kk;
      sum += v;
      mx = max(mx, v);
    }
    // wave reductions by DPP rotations and lane reads (no LDS round trips: the search
    // below takes a dozen of them in a row)
    sum = static_cast<int>(wave_sum_u32(static_cast<uint32_t>(sum)));
    mx = static_cast<int>(wave_max_u32(static_cast<uint32_t>(mx)));
    auto runs_of = [&](int v, int c, float rc) { return v <= c ? 1 : ceil_div_small(v, c, rc); };
    auto pieces = [&](int c) {   // runs over all pairs at run length c (wave-uniform)
      const float rc = __builtin_amdgcn_rcpf(static_cast<float>(c));   // within 1 ulp
      int t = 0;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (i < ni && lane + kWave * i < a.B) t += runs_of(nb[i], c, rc);
      return static_cast<int>(wave_sum_u32(static_cast<uint32_t>(t))) * Hkv;
    };
    // smallest c in [lo, hi] with pieces(c) <= resident workgroups (pieces is
    // non-increasing in c; at c = mx every pair is one run), at least what num_splits
    // runs need for the longest request and at most the kMaxDenseBlocks a workgroup
    // stages (the caller guarantees ceil(max_blocks / num_splits) fits)
    const int full = max(a.target_wgs, 1);
    const int need = max((mx + S - 1) / S, 1);
    const int64_t even = (static_cast<int64_t>(sum) * Hkv + full - 1) / full;
    int lo = static_cast<int>(max<int64_t>(need, min<int64_t>(even, kMaxDenseBlocks)));
    int hi = max(min(mx, kMaxDenseBlocks), lo);
    // pieces(c) <= sum * Hkv / c + pairs, so c = ceil(sum * Hkv / (full - pairs)) fits
    const int pairs = a.B * Hkv;
    if (full > pairs) {
      const int64_t fit = (static_cast<int64_t>(sum) * Hkv + (full - pairs) - 1) / (full - pairs);
      hi = max(lo, static_cast<int>(min<int64_t>(hi, max<int64_t>(fit, 1))));
    }
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (pieces(mid) <= full) hi = mid;
      else lo = mid + 1;
    }
    const int c = lo;
    const float rc = __builtin_amdgcn_rcpf(static_cast<float>(c));
    int k[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) k[i] = runs_of(nb[i], c, rc);
    // level j holds the pairs of the requests with more than j runs
    int base = 0, j = -1, idx = 0;
    for (int jj = 0; jj < S; ++jj) {
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < NI; ++i) cnt += (i < ni && lane + kWave * i < a.B && k[i] > jj) ? 1 : 0;
      cnt = static_cast<int>(wave_sum_u32(static_cast<uint32_t>(cnt)));
      if (cnt == 0) break;
      if (lin < base + cnt * Hkv) {
        j = jj;
        idx = lin - base;
        break;
      }
      base += cnt * Hkv;
    }
    if (lane == 0) lds[0] = j;
    if (j >= 0) {
      // the (idx / Hkv)-th request (in index order) with more than j runs
      const int want = idx / Hkv;
      int seen = 0;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bool f = i < ni && lane + kWave * i < a.B && k[i] > j;
        const uint64_t m = __ballot(f);
        const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
        if (f && seen + below == want) {
          const int sz = (nb[i] + k[i] - 1) / k[i];
          const int first = j * sz;
          lds[1] = lane + kWave * i;
          lds[2] = idx - want * Hkv;
          lds[3] = first;
          lds[4] = max(0, min(nb[i], first + sz) - first);
          lds[5] = k[i];
          lds[6] = row0s[i];
          lds[7] = qos[i];
          lds[8] = kvs[i];
        }
        seen += __builtin_popcountll(m);
      }
    }
  }
  __syncthreads();
  pc.j = lds[0];
  if (pc.j < 0) return false;
  pc.r = lds[1];
  pc.h = lds[2];
  pc.first = lds[3];
  pc.n = lds[4];
  pc.k = lds[5];
  pc.row0 = lds[6];
  pc.qo = lds[7];
  pc.kv = lds[8];
  return true;
}

// The plan with as few request slots a lane as the batch needs (the slots are unrolled).
__device__ inline bool dense_compact_piece(const AttnArgs& a, int max_blocks, int* lds,
                                           DensePiece& pc) {
  static_assert(kCompactMaxRequests == 8 * kWave, "slot counts below");
  if (a.B <= kWave) return dense_compact_piece_t<1>(a, max_blocks, lds, pc);
  if (a.B <= 2 * kWave) return dense_compact_piece_t<2>(a, max_blocks, lds, pc);
  return dense_compact_piece_t<8>(a, max_blocks, lds, pc);
}

// Where the 32-token blocks of a (request, KV head) come from.
enum SourceMode : int {
  kSrcView = 0,     // dense, through the P32 sub-page view of the draft layer
  kSrcSparse = 1,   // sparse: the union of the P128 pages the tokens selected
  kSrcPaged = 2,    // dense over ordinary head-major P128 pages and a block table
  kSrcSparseSelect = 3,  // sparse, each token's pages chosen in the kernel from page scores
  kSrcSparseSelectWide = 4,  // the same, tokens with wide tables selecting by the bit search
};

__host__ __device__ constexpr bool is_select(int mode) {
  return mode == kSrcSparseSelect || mode == kSrcSparseSelectWide;
}

__host__ __device__ constexpr bool is_sparse(int mode) {
  return mode == kSrcSparse || is_select(mode);
}

// Per dense split: for kSrcView the P32 page index of each block's K sub-page (the view
// puts V one P128 page, four P32 pages, after K); for kSrcPaged the physical P128 page
// of each block.  -1 marks an index outside the pool.
struct DenseMeta {
  int32_t x[kMaxDenseBlocks];
};

// The block list of one workgroup's split, staged in LDS before any asynchronous copy
// (a vector load of block metadata inside the copy pipeline would wait behind every
// copy in flight), then read back one block ahead of use and resolved into scalar
// addresses.
template <int MODE, int D, int KDT>
struct BlockList {
  using Gm = Geo<D, KDT>;
  using Lds = typename std::conditional<is_sparse(MODE), UnionLds, DenseMeta>::type;
  struct Raw {
    int a, b, c;
  };
  int base;    // first block (dense) or union entry (sparse) of the split
  int nblk;    // blocks of the split

  // All 256 threads call.  Sparse: the union of the pages the request's tokens chose,
  // cut into num_splits near-equal runs.  Dense: runs of one length for the whole call.
  __device__ __forceinline__ void stage(Lds& ul, int* chunk_lds, const AttnArgs& a,
                                        const DenseSource& ds, const SparseSource& ss, int r,
                                        int h, int split, int row0, int qo, int kv) {
    if constexpr (is_sparse(MODE)) {
      const int n_union = build_union<is_select(MODE), MODE == kSrcSparseSelectWide>(ul, ss, r, h, a.num_kv_heads, row0, qo, kv, a.dev_err,
                                      split == 0);
      const int chunk = (n_union + a.num_splits - 1) / a.num_splits;
      base = split * chunk;
      nblk = 4 * max(0, min(n_union, base + chunk) - base);
    } else {
      const int cap = MODE == kSrcView ? ds.max_sub_pages : 4 * ss.max_pages;
      const int chunk = dense_chunk(a, cap, chunk_lds);
      const int nb = (kv + kSub - 1) / kSub;
      const int first = split * chunk;
      stage_range(ul, a, ds, ss, r, first, max(0, min(nb, first + chunk) - first));
    }
  }

  // Dense only: blocks [first, first + n) of request r, n <= kMaxDenseBlocks.  Every
  // block's page index is checked against the pool (out of range: flagged, and the block
  // is read masked out).  All 256 threads call; ends with a barrier.
  __device__ __forceinline__ void stage_range(Lds& ul, const AttnArgs& a, const DenseSource& ds,
                                              const SparseSource& ss, int r, int first, int n) {
    static_assert(!is_sparse(MODE), "dense block lists only");
    const int tid = threadIdx.x;
    base = first;
    nblk = n;
    if constexpr (MODE == kSrcView) {
      for (int b = tid; b < nblk; b += 256) {
        int64_t xk, xv;
        const bool ok = view_pages(ds, r, base + b, xk, xv) && xv == xk + 4;
        if (!ok) set_err(a.dev_err, SDV_DEVERR_PAGE_RANGE);
        ul.x[b] = ok ? static_cast<int32_t>(xk) : -1;
      }
    } else {
      const int32_t* bt = ss.block_table + static_cast<int64_t>(r) * ss.bt_stride;
      for (int b = tid; b < nblk; b += 256) {
        const int32_t phys = bt[(base + b) >> 2];
        const bool ok = phys >= 0 && phys < ss.num_pages;
        if (!ok) set_err(a.dev_err, SDV_DEVERR_PAGE_RANGE);
        ul.x[b] = ok ? phys : -1;
      }
    }
    __syncthreads();
  }

  // Metadata of split-local block b as stored (wave-uniform values in vector registers).
  __device__ __forceinline__ Raw fetch(const Lds& ul, int b) const {
    Raw m;
    if constexpr (is_sparse(MODE)) {
      const int e = base + (b >> 2);
      m.a = ul.upage[e];
      m.b = ul.uphys[e];
      m.c = ul.umask[e];
    } else {
      m.a = ul.x[b];
      m.b = m.c = 0;
    }
    return m;
  }

  // Block b's K and V byte addresses, first position and the verify tokens it serves, in
  // scalar registers.  A block whose page index was out of range reads page 0 masked out.
  __device__ __forceinline__ void resolve(const Raw& m, int b, int h, int Hkv,
                                          const DenseSource& ds, const SparseSource& ss,
                                          uint64_t& kbase, uint64_t& vbase, int& pos0,
                                          int& mask) const {
    if constexpr (is_sparse(MODE)) {
      const int quarter = b & 3;
      const int p = __builtin_amdgcn_readfirstlane(m.a);
      const int phys = __builtin_amdgcn_readfirstlane(m.b);
      mask = __builtin_amdgcn_readfirstlane(m.c);
      pos0 = p * kPage + quarter * kSub;
      const uint64_t off = static_cast<uint64_t>(
          (static_cast<int64_t>(phys) * ss.page_stride +
           (static_cast<int64_t>(h) * kPage + quarter * kSub) * D) * Gm::EB);
      kbase = reinterpret_cast<uint64_t>(ss.k) + off;
      vbase = reinterpret_cast<uint64_t>(ss.v) + off;
    } else if constexpr (MODE == kSrcView) {
      int64_t xk = __builtin_amdgcn_readfirstlane(m.a);
      mask = xk < 0 ? 0 : ~0;
      xk = xk < 0 ? 0 : xk;
      const int64_t xv = xk + 4;
      pos0 = (base + b) * kSub;
      kbase = reinterpret_cast<uint64_t>(ds.root) +
              static_cast<uint64_t>((xk * Hkv + h) * kSub * D * Gm::EB);
      vbase = reinterpret_cast<uint64_t>(ds.root) +
              static_cast<uint64_t>((xv * Hkv + h) * kSub * D * Gm::EB);
    } else {
      int64_t phys = __builtin_amdgcn_readfirstlane(m.a);
      mask = phys < 0 ? 0 : ~0;
      phys = phys < 0 ? 0 : phys;
      const int blk = base + b;
      pos0 = blk * kSub;
      const uint64_t off = static_cast<uint64_t>(
          (phys * ss.page_stride + (static_cast<int64_t>(h) * kPage + (blk & 3) * kSub) * D) *
          Gm::EB);
      kbase = reinterpret_cast<uint64_t>(ss.k) + off;
      vbase = reinterpret_cast<uint64_t>(ss.v) + off;
    }
  }
};


// Persistent split-KV partition for dense sources ("stream-K"): the (request, KV head)
// pairs, request-major, laid end to end form one list of W 32-token blocks, and
// workgroup g attends blocks [g L, (g + 1) L) of it, so every workgroup has the same
// amount of work whatever the spread of kv_len.  A piece of a pair inside the range is
// written as the partial of split slot (g - first workgroup of the pair); the workgroup
// that ends a pair writes lse = -inf into the pair's later slots, so the combine sees
// exactly num_splits slots per row.  L >= ceil(max blocks of a request / (num_splits -
// 1)), so no pair spans more than num_splits workgroups, and L <= kMaxDenseBlocks.
// Requests with inconsistent lengths count as empty (workgroup 0 flags them).
struct PersistLds {
  int cum[kPersistMaxRequests + 1];   // blocks per request, then their exclusive prefix
  int seg_len;
};

// All 256 threads call.  Fills pl.cum with the exclusive prefix of every request's
// 32-token block count (cum[B] = total; inconsistent requests count 0 and workgroup 0
// flags them) and pl.seg_len with the range length L.  Ends with a barrier.
template <int MODE>
__device__ __forceinline__ void persistent_prefix(PersistLds& pl, const AttnArgs& a,
                                                  const DenseSource& ds, const SparseSource& ss) {
  const int tid = threadIdx.x;
  const int Hkv = a.num_kv_heads;
  const int S = a.num_splits;
  const int cap = MODE == kSrcView ? ds.max_sub_pages : 4 * ss.max_pages;
  const int64_t kv_cap = static_cast<int64_t>(cap) * kSub;
  for (int rr = tid; rr < a.B; rr += 256) {
    const int row0 = a.qo_indptr[rr];
    const int qo = a.qo_indptr[rr + 1] - row0;
    const int kv = a.kv_len[rr];
    const bool bad_len = qo < 1 || qo > a.max_qo_len || kv < qo || row0 < 0 ||
                         static_cast<int64_t>(row0) + qo > static_cast<int64_t>(a.B) * a.max_qo_len;
    const bool bad_cap = !bad_len && kv > kv_cap;
    if ((bad_len || bad_cap) && blockIdx.x == 0)
      set_err(a.dev_err, bad_len ? SDV_DEVERR_QO_LEN : SDV_DEVERR_KV_CAPACITY);
    pl.cum[rr] = bad_len || bad_cap ? 0 : (kv + kSub - 1) / kSub;
  }
  __syncthreads();
  if (tid < kWave) {
    // exclusive prefix of the block counts in place (cum[B] = total), their maximum, and
    // the range length L
    int run = 0, mx = 0;
    for (int c = 0; c < a.B; c += kWave) {
      const int rr = c + tid;
      const int v = rr < a.B ? pl.cum[rr] : 0;
      int inc = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_up(inc, off, kWave);
        if (tid >= off) inc += t;
      }
      if (rr < a.B) pl.cum[rr] = run + inc - v;
      run += __shfl(inc, kWave - 1, kWave);
      mx = max(mx, v);
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) mx = max(mx, __shfl_xor(mx, off, kWave));
    if (tid == 0) {
      pl.cum[a.B] = run;
      const int64_t work = static_cast<int64_t>(run) * Hkv;
      const int64_t wgs = a.target_wgs > 0 ? a.target_wgs : 1;
      int64_t len = max<int64_t>((work + wgs - 1) / wgs, (mx + S - 2) / (S - 1));
      len = min<int64_t>(max<int64_t>(len, 1), kMaxDenseBlocks);
      pl.seg_len = static_cast<int>(len);
    }
  }
  __syncthreads();
}

// The request holding flat block `pos` (< W): the last r with Hkv * cum[r] <= pos (it is
// not empty).  Wave-uniform.
__device__ __forceinline__ int persistent_request(const PersistLds& pl, int B, int Hkv, int pos) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(pl.cum[mid]) * Hkv <= pos) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// All 256 threads call.  attend(r, h, row0, qo, kv, first, n, slot) attends blocks
// [first, first + n) of pair (r, h) into split slot `slot`; a barrier follows each call.
template <int MODE, class Attend>
__device__ __forceinline__ void persistent_walk(PersistLds& pl, const AttnArgs& a,
                                                const DenseSource& ds, const SparseSource& ss,
                                                Attend&& attend) {
  const int tid = threadIdx.x;
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int S = a.num_splits;
  persistent_prefix<MODE>(pl, a, ds, ss);
  // values read from LDS are uniform: keep them in scalar registers
  const int L = __builtin_amdgcn_readfirstlane(pl.seg_len);
  const int W = __builtin_amdgcn_readfirstlane(pl.cum[a.B]) * Hkv;
  const int g = blockIdx.x;
  if (static_cast<int64_t>(g) * L >= W) return;
  const int begin = g * L;
  const int end = static_cast<int>(min<int64_t>(static_cast<int64_t>(begin) + L, W));
  int r = persistent_request(pl, a.B, Hkv, begin);
  int pos = begin;
  const int64_t rows_cap = static_cast<int64_t>(a.B) * a.max_qo_len;
  while (pos < end) {
    const int c0 = __builtin_amdgcn_readfirstlane(pl.cum[r]);
    const int nb = __builtin_amdgcn_readfirstlane(pl.cum[r + 1]) - c0;
    const int rstart = c0 * Hkv;
    if (nb == 0 || pos >= rstart + nb * Hkv) {
      ++r;
      continue;
    }
    const int h = (pos - rstart) / nb;
    const int pstart = rstart + h * nb;
    const int pend = pstart + nb;
    const int stop = min(end, pend);
    const int slot = g - pstart / L;
    const int row0 = a.qo_indptr[r];
    const int qo = a.qo_indptr[r + 1] - row0;
    const int kv = a.kv_len[r];
    attend(r, h, row0, qo, kv, pos - pstart, stop - pos, slot);
    if (stop == pend) {
      // the pair ends here: its later split slots hold no keys
      const int rows = qo * G;
      for (int e = tid; e < (S - 1 - slot) * rows; e += 256) {
        const int k = slot + 1 + e / rows;
        const int row = e % rows;
        const int t = row / G;
        a.part_lse[(k * rows_cap + row0 + t) * a.num_q_heads + h * G + (row - t * G)] = -INFINITY;
      }
    }
    __syncthreads();   // LDS is reused by the next piece
    pos = stop;
  }
}

}  // namespace
}  // namespace sdv
