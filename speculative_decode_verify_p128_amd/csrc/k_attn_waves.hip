// Verify attention on the CDNA4 matrix cores, one block stream per wave (bf16 queries;
// bf16 or fp8 K/V).
//
// What is computed: token t of request r, query head hq of KV head h attends the
// positions j < bound(r,t) = kv_len - qo_len + t + 1 ("[TRTLLM-14093][feat] Eagle3
// for M3 MSA path + CUDA graphs compatibility", MSA verify commit); dense keys come
// through the P32 sub-page view of the draft layer's P128 pages ("[None][perf]
// Default Minimax-m3 to unified draft-target kv manager ...", Description and item 2
// Grouped-HND), sparse keys only from the pages the token selected.  Float32
// accumulation; probabilities enter the value product as bf16.
//
// Work layout (gfx950, wave64, v_mfma_f32_16x16x32_bf16):
//   * One workgroup (4 waves) per (request, KV head, split).  Every wave holds all the
//     query rows of the (request, KV head) — G x qo (token, head) pairs, row = t * G + g,
//     in RT tiles of 16 — and takes every fourth 32-token block of the split.  Each K/V
//     byte is therefore copied into LDS once and read from LDS once, by one wave, and a
//     wave keeps its own online-softmax state; the waves never wait for each other until
//     the end.
//   * A wave streams its blocks through a private two-slot LDS ring with asynchronous
//     global->LDS copies (global_load_lds_dwordx4, non-temporal): while a block is
//     computed the next two are in flight.  Its waits are its own vmcnt / lgkmcnt waits;
//     there is no workgroup barrier in the block loop.
//   * Scores are computed transposed (S^T = K Q^T) for every row tile from one read of
//     the K block, and one read and transpose of the V block serves the value product
//     of every row tile (O^T += V^T P^T).
//   * At the end the four waves' (max, sum, output) merge in a fixed order through LDS,
//     and wave 0 writes the rows (or a normalised partial and its log-sum-exp for the
//     split-KV combine) straight from registers: each lane holds a contiguous quarter of
//     a row's channels.
#include "mfma_attn.h"
#include "sparse_union.h"

namespace sdv {
namespace {

constexpr int kWaveSlots = 2;   // ring slots per wave

// One wave's copy of a whole 32-token block (K then V) into a ring slot: 32 / RPI
// asynchronous 16-byte-per-lane loads per half.  Lane l of instruction n lands at
// half + (n * 64 + l) * 16, which is LDS row n * RPI + l / CPR, chunk l % CPR of the
// swizzled block; the lane reads the global chunk that belongs there (Geo::src).
template <int D, int KDT>
struct WaveCopier {
  using Gm = Geo<D, KDT>;
  static constexpr int PER_HALF = 32 / Gm::RPI;
  static constexpr int NI = 2 * PER_HALF;        // loads per block
  uint32_t off[PER_HALF];

  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int n = 0; n < PER_HALF; ++n) {
      off[n] = static_cast<uint32_t>(Gm::src(n * Gm::RPI + lane / Gm::CPR, lane % Gm::CPR));
    }
  }

  // kbase, vbase: first byte of the block's K and V runs; slot_lds: LDS address of the
  // slot.  All three are wave-uniform.
  __device__ __forceinline__ void issue(uint64_t kbase, uint64_t vbase, uint32_t slot_lds) const {
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
      const uint64_t base = hv ? vbase : kbase;
#pragma unroll
      for (int n = 0; n < PER_HALF; ++n) {
        const uint32_t m0 = slot_lds + hv * Gm::HALF + n * 1024;
        // Inline assembly, so that the compiler's wait insertion, which cannot tell ring
        // slots apart, does not drain the copies in flight; this wave's own vmcnt waits
        // order copies and reads.  M0 holds the copy's LDS base.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     :
                     : "s"(m0), "v"(off[n]), "s"(base)
                     : "memory", "m0");
#pragma clang diagnostic pop
      }
    }
  }
};

// Merge buffer slot of (row, 16-byte piece k of the row): pieces are XOR-swizzled by a
// key of the row (row_key16), as the K/V rows are, since lane (i, q) accesses piece
// q * D/16 + k of row i: the same lane-to-bank-group pattern as the K operand reads.
template <int D>
__device__ __forceinline__ int merge_index(int row, int k) {
  return row * (D / 4) + (k ^ row_key16(row & 15));
}

// LDS of the per-wave kernels: the four waves' rings (the merge regions reuse them), the
// waves' row maxima and sums, and the staged block list.
template <int RT, int D, int KDT, int MODE>
struct WavesLds {
  using Gm = Geo<D, KDT>;
  static constexpr int ROWS = RT * 16;
  static constexpr int WAVE_RING = kWaveSlots * Gm::BLOCK;
  static constexpr int RING = 4 * WAVE_RING;
  static_assert(2 * ROWS * D * 4 <= RING, "merge regions reuse the ring");
  __attribute__((aligned(16))) char ring[RING];
  float M[4][ROWS];
  float L[4][ROWS];
  typename BlockList<MODE, D, KDT>::Lds ul;
  int chunk;
};

// Attention of the G x qo query rows of (request r, KV head h) over the staged block
// range `bl` (whose metadata sits in sh.ul): every wave streams every fourth block, then
// the waves merge and wave 0 writes the rows (out_slot < 0) or the normalised partial and
// log-sum-exp into split slot out_slot.  All 256 threads call; LDS is free again only
// after a barrier that follows the call.
template <int RT, int D, int KDT, int MODE>
__device__ __forceinline__ void waves_attend(WavesLds<RT, D, KDT, MODE>& sh, const AttnArgs& a,
                                             const DenseSource& ds, const SparseSource& ss,
                                             const BlockList<MODE, D, KDT>& bl, int r, int h,
                                             int row0, int qo, int kv, int out_slot) {
  using Gm = Geo<D, KDT>;
  using Cp = WaveCopier<D, KDT>;
  using BL = BlockList<MODE, D, KDT>;
  constexpr int STEPS = Gm::STEPS;
  constexpr int NT = Gm::NT;
  constexpr int ROWS = RT * 16;
  constexpr int A = kWaveSlots;
  constexpr int WAVE_RING = A * Gm::BLOCK;
  static_assert(D / 4 <= 32 && (D / 4) % 8 == 0, "a lane's quarter row");
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i = lane & 15;
  const int q = lane >> 4;
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int nrows = qo * G;

  // This lane's query row of every row tile (lane i of the tile), its token and bound
  // (the rows' query values load after the first copies are issued, below).
  int t_row[RT], bound_row[RT];
  bf16x8 qb[RT][STEPS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + i;
    const bool live = row < nrows;
    t_row[rt] = live ? row / G : 0;
    bound_row[rt] = live ? kv - qo + t_row[rt] + 1 : 0;
  }
  const float qk_scale = a.softmax_scale * a.k_scale * kLog2e;

  // This wave's blocks: split-local b = wave + 4 j, j < nbw.
  const int nblk = bl.nblk;
  const int nbw = nblk > wave ? (nblk - wave + 3) / 4 : 0;

  auto fetch = [&](int b) { return bl.fetch(sh.ul, b); };
  auto resolve = [&](const typename BL::Raw& m, int b, uint64_t& kbase, uint64_t& vbase, int& pos0,
                     int& mask) { bl.resolve(m, b, h, Hkv, ds, ss, kbase, vbase, pos0, mask); };

  Cp copier;
  copier.init(lane);
  char* wring = sh.ring + wave * WAVE_RING;
  const uint32_t wring_lds = lds_address(wring);
  const int all_tokens = qo >= 32 ? ~0 : (1 << qo) - 1;
  const int first_bound = kv - qo + 1;

  f32x4 o[RT][NT];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int n = 0; n < NT; ++n) o[rt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
  }

  int slot_pos[A], slot_mask[A];
#pragma unroll
  for (int u = 0; u < A; ++u) {
    slot_pos[u] = slot_mask[u] = 0;
    if (u < nbw) {
      uint64_t kb, vb;
      resolve(fetch(wave + 4 * u), wave + 4 * u, kb, vb, slot_pos[u], slot_mask[u]);
      copier.issue(kb, vb, wring_lds + u * Gm::BLOCK);
    }
  }
  typename BL::Raw next{0, 0, 0};
  if (A < nbw) next = fetch(wave + 4 * A);

  // The query rows load while the first blocks' copies are in flight; one wait then
  // covers both, so no wait inside the block loop has to account for Q (the compiler,
  // which does not see the copies, would otherwise wait for everything in flight there).
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + i;
    const bool live = row < nrows;
    const int g_row = live ? row - t_row[rt] * G : 0;
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(row0 + t_row[rt]) * a.num_q_heads + h * G + g_row) * D +
                      q * (D / 4)) * 2;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const uint4 w = live ? *reinterpret_cast<const uint4*>(qp + Gm::step_unit(q, s) * 16)
                           : make_uint4(0, 0, 0, 0);
      qb[rt][s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  auto step = [&](auto slot_c, int j) {
    constexpr int u = decltype(slot_c)::value;
    // This wave's copies of block j have landed (those of later blocks may not have).
    wait_blocks<Cp::NI, A - 1>(min(nbw - 1 - j, A - 1));
    const char* kb = wring + u * Gm::BLOCK;
    const char* vb = kb + Gm::HALF;
    bf16x8 kop[2][STEPS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < STEPS; ++s) kop[tt][s] = k_operand<D, KDT>(kb, tt, s, i, q);
    uint32_t vraw[8][4];
    v_runs<D, KDT, NT>(vb, i, q, 0, vraw);
    const int pos0 = slot_pos[u];
    const int mask = slot_mask[u];
    // The slot's reads have returned: refill it with block j + A.
    wait_lgkmcnt0();
    if (j + A < nbw) {
      const int bn = wave + 4 * (j + A);
      uint64_t kbn, vbn;
      resolve(next, bn, kbn, vbn, slot_pos[u], slot_mask[u]);
      copier.issue(kbn, vbn, wring_lds + u * Gm::BLOCK);
      if (j + A + 1 < nbw) next = fetch(bn + 4);
    }
    const bool inside = pos0 + kSub <= first_bound && (mask & all_tokens) == all_tokens;

    // Row tiles one at a time: scores S^T (unscaled), the lazy rescale and the
    // probabilities, so that only one tile's scores are live.  A row's reference maximum
    // moves only when a score passes it by more than 2^8 (probabilities stay <= 256); the
    // cross-lane maximum runs only when some lane's partial maximum passed it.  The
    // scale is positive, so it commutes with max.  Masked scores are -inf and give 0; a
    // row with no live score yet keeps m = -inf and has only masked scores here.
    bf16x8 pb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 sacc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) sacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < STEPS; ++s)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) sacc[tt] = mfma16(kop[tt][s], qb[rt][s], sacc[tt]);
      float mx = -INFINITY;
      if (inside) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[tt][e]);
      } else {
        const int bnd = ((mask >> t_row[rt]) & 1) ? bound_row[rt] : 0;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int pos = pos0 + tt * 16 + 4 * q + e;
            const float sv = pos < bnd ? sacc[tt][e] : -INFINITY;
            sacc[tt][e] = sv;
            mx = fmaxf(mx, sv);
          }
      }
      const float ms = mx * qk_scale;
      if (__any(ms > m_run[rt] + kRescaleLog2)) {
        float mr = fmaxf(ms, __shfl_xor(ms, 16, kWave));
        mr = fmaxf(mr, __shfl_xor(mr, 32, kWave));
        if (mr > m_run[rt] + kRescaleLog2) {
          const float alpha = m_run[rt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[rt] - mr);
          l_run[rt] *= alpha;
#pragma unroll
          for (int n = 0; n < NT; ++n) o[rt][n] *= alpha;
          m_run[rt] = mr;
        }
      }
      const float m_use = m_run[rt] == -INFINITY ? 0.f : m_run[rt];
      float p[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[0][e], qk_scale, -m_use));
        p[e + 4] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[1][e], qk_scale, -m_use));
      }
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ls += p[e];
      l_run[rt] += ls;
      pb[rt] = __builtin_bit_cast(
          bf16x8, make_uint4(pack2_bf16(p[0], p[1]), pack2_bf16(p[2], p[3]),
                             pack2_bf16(p[4], p[5]), pack2_bf16(p[6], p[7])));
    }
    // value product; positions past kv_len read as 0 (stale storage must not reach P * V)
    if (pos0 + kSub > kv) v_zero_tail(q, pos0, kv, vraw);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const bf16x8 vop = v_operand<KDT>(vraw, n);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) o[rt][n] = mfma16(vop, pb[rt], o[rt][n]);
    }
  };

  for (int j0 = 0; j0 < nbw; j0 += A) {
    static_for<A>([&](auto slot_c) {
      const int j = j0 + decltype(slot_c)::value;
      if (j < nbw) step(slot_c, j);
    });
  }
  wait_vmcnt<0>();

  // ---- merge the four waves: reference max, sums, outputs (fixed order) ----
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l_run[rt] += __shfl_xor(l_run[rt], 16, kWave);
    l_run[rt] += __shfl_xor(l_run[rt], 32, kWave);
    if (q == 0) {
      sh.M[wave][rt * 16 + i] = m_run[rt];
      sh.L[wave][rt * 16 + i] = l_run[rt];
    }
  }
  __syncthreads();   // every wave is done with its ring; M and L are visible
  float m_ref[RT], l_tot[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + i;
    float mref = sh.M[0][row];
#pragma unroll
    for (int w = 1; w < 4; ++w) mref = fmaxf(mref, sh.M[w][row]);
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sh.M[w][row];
      lt += mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mref) * sh.L[w][row];
    }
    m_ref[rt] = mref;
    l_tot[rt] = lt;
    const float f = m_run[rt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[rt] - mref);
#pragma unroll
    for (int n = 0; n < NT; ++n) o[rt][n] *= f;
  }
  // Piece k = 4 n' ... of a lane: element e of tile n is channel NT * (4q + e) + n; the
  // lane's 4 NT values form the contiguous channels q * D/4 .. q * D/4 + D/4 - 1, kept
  // as D/16 pieces of 4 floats: piece k holds channels q * D/4 + 4k .. + 3.
  float4* reg0 = reinterpret_cast<float4*>(sh.ring);
  float4* reg1 = reg0 + ROWS * D / 4;
  auto lane_piece = [&](int rt, int k) {
    // channels c = q*D/4 + 4k + c4, c4 = 0..3  ->  (e, n) with NT*(4q+e) + n = c
    float4 v;
    float* vv = reinterpret_cast<float*>(&v);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int c = 4 * k + c4;        // 0 .. D/4 - 1 within the lane's quarter
      vv[c4] = o[rt][c % NT][c / NT];
    }
    return v;
  };
  auto add_piece = [&](int rt, int k, const float4& v) {
    const float* vv = reinterpret_cast<const float*>(&v);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int c = 4 * k + c4;
      o[rt][c % NT][c / NT] += vv[c4];
    }
  };
  constexpr int KP = D / 16;   // pieces per lane per row
  auto put = [&](float4* region) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int k = 0; k < KP; ++k)
        region[merge_index<D>(rt * 16 + i, q * KP + k)] = lane_piece(rt, k);
  };
  auto take = [&](const float4* region) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int k = 0; k < KP; ++k) add_piece(rt, k, region[merge_index<D>(rt * 16 + i, q * KP + k)]);
  };
  // (w0 + w1) + (w2 + w3)
  if (wave == 1) put(reg0);
  if (wave == 3) put(reg1);
  __syncthreads();
  if (wave == 0) take(reg0);
  if (wave == 2) take(reg1);
  __syncthreads();
  if (wave == 2) put(reg0);
  __syncthreads();
  if (wave != 0) return;
  take(reg0);

  // ---- wave 0 writes: its lane holds channels q*D/4 .. +D/4-1 of row rt*16 + i ----
  const int64_t rows_cap = static_cast<int64_t>(a.B) * a.max_qo_len;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + i;
    if (row >= nrows) continue;
    const int t = row / G;
    const int g = row - t * G;
    const int hq = h * G + g;
    const int64_t qrow = row0 + t;
    const float L = l_tot[rt];
    const float inv = L > 0.f ? a.v_scale / L : 0.f;
    float v[D / 4];
#pragma unroll
    for (int c = 0; c < D / 4; ++c) v[c] = o[rt][c % NT][c / NT] * inv;
    const int c0 = q * (D / 4);
    if (out_slot < 0) {
      const int64_t idx = (qrow * a.num_q_heads + hq) * D + c0;
      if (a.out_dt == SDV_BF16) {
        uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + idx);
#pragma unroll
        for (int c = 0; c < D / 4; c += 8)
          dst[c / 8] = make_uint4(pack2_bf16(v[c], v[c + 1]), pack2_bf16(v[c + 2], v[c + 3]),
                                  pack2_bf16(v[c + 4], v[c + 5]), pack2_bf16(v[c + 6], v[c + 7]));
      } else {
        float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + idx);
#pragma unroll
        for (int c = 0; c < D / 4; c += 4) dst[c / 4] = make_float4(v[c], v[c + 1], v[c + 2], v[c + 3]);
      }
    } else {
      // A row with no live position (an empty split) leaves its partial output unwritten:
      // the combine skips rows whose log-sum-exp is -inf.
      const int64_t unit = (static_cast<int64_t>(out_slot) * rows_cap + qrow) * a.num_q_heads + hq;
      if (L > 0.f) {
        float4* dst = reinterpret_cast<float4*>(a.part_o + unit * D + c0);
#pragma unroll
        for (int c = 0; c < D / 4; c += 4) dst[c / 4] = make_float4(v[c], v[c + 1], v[c + 2], v[c + 3]);
      }
      if (q == 0) a.part_lse[unit] = L > 0.f ? (m_ref[rt] + __log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

// Waves per SIMD an instantiation may share a CU with: 16-row tiles whose LDS leaves room
// for a second workgroup (fp8 K/V or head_dim 64) run two workgroups per CU, so a grid of
// up to twice the CU count (many splits) is resident at once; the others keep the whole
// register file (up to 512 registers per lane) at one workgroup per CU.
template <int RT, int D, int KDT, int MODE>
constexpr int waves_occupancy() {
  return RT == 1 && sizeof(WavesLds<RT, D, KDT, MODE>) <= 80 * 1024 ? 2 : 1;
}

// Requests a launch may order by work, and the largest work key (qo_len x top_k <= 512).
constexpr int kOrderMaxRequests = 1024;
constexpr int kOrderKeys = 512;

// LDS of the ordering step (inside the ring, not yet in use when it runs).
struct OrderLds {
  int row0[kOrderMaxRequests];
  int qo[kOrderMaxRequests];
  int kv[kOrderMaxRequests];
  int key[kOrderMaxRequests];
  int hist[kOrderKeys];
  int start[kOrderKeys];      // requests with a larger key (or equal key, lower bin)
  int wave_tot[256 / kWave];
  int pick[2];
};

// Exclusive prefix over the workgroup of one int per thread (thread order), with the
// total: lane shuffles inside each wave, then the four wave totals.  All threads call;
// two barriers.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += t;
  }
  if (lane == kWave - 1) wave_tot[wv] = inc;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int k = 0; k < 256 / kWave; ++k) {
    const int tw = wave_tot[k];
    base += k < wv ? tw : 0;
    total += tw;
  }
  __syncthreads();
  return base + inc - v;
}

// The request that grid position pos takes when the requests are ordered longest first:
// by the pages their tokens can select, min(valid pages, qo_len x top_k) (inconsistent
// requests count 0), ties by index.  With more (request, KV head) workgroups than the GPU
// holds at once, the long ones then start in the first generation and the short ones
// fill the last.  Every workgroup derives the same order from the lengths: a histogram
// of the keys, its prefix from the largest key down, the key bin that holds position
// pos, then the requests of that bin in index order.  The request's lengths are returned
// from the same loads.  All threads call.
__device__ int request_by_work(OrderLds& o, const AttnArgs& a, const SparseSource& ss, int pos,
                               int& row0, int& qo, int& kv) {
  const int tid = threadIdx.x;
  const int B = a.B;
  for (int k = tid; k < kOrderKeys; k += 256) o.hist[k] = 0;
  for (int i = tid; i < B; i += 256) {
    const int r0 = a.qo_indptr[i];
    const int q = a.qo_indptr[i + 1] - r0;
    const int k = a.kv_len[i];
    o.row0[i] = r0;
    o.qo[i] = q;
    o.kv[i] = k;
    // any lengths give a key in [0, kOrderKeys): the kernel's own checks reject the
    // inconsistent ones later
    const bool ok = q >= 1 && q <= a.max_qo_len && k >= q;
    const int pages = k / kPage + (k % kPage != 0);
    o.key[i] = ok ? min(min(pages, q * ss.top_k), kOrderKeys - 1) : 0;
  }
  __syncthreads();
  for (int i = tid; i < B; i += 256) atomicAdd(&o.hist[o.key[i]], 1);
  __syncthreads();
  // start[k] = requests with key > k: thread t owns keys 511 - 2t and 510 - 2t
  static_assert(kOrderKeys == 2 * 256, "two key bins a thread");
  const int k_hi = kOrderKeys - 1 - 2 * tid;
  const int c0 = o.hist[k_hi];
  const int c1 = o.hist[k_hi - 1];
  int total;
  const int excl = block_exclusive_scan(c0 + c1, o.wave_tot, total);
  o.start[k_hi] = excl;
  o.start[k_hi - 1] = excl + c0;
  if (pos >= excl && pos < excl + c0) o.pick[0] = k_hi;
  if (pos >= excl + c0 && pos < excl + c0 + c1) o.pick[0] = k_hi - 1;
  __syncthreads();
  const int ks = o.pick[0];
  const int m = pos - o.start[ks];
  // the m-th request (by index) whose key is ks: thread t holds indices 4t .. 4t + 3
  static_assert(kOrderMaxRequests == 4 * 256, "four requests a thread");
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * tid + j;
    cnt += i < B && o.key[i] == ks;
  }
  int unused;
  int before = block_exclusive_scan(cnt, o.wave_tot, unused);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * tid + j;
    if (i < B && o.key[i] == ks) {
      if (before == m) o.pick[1] = i;
      ++before;
    }
  }
  __syncthreads();
  const int r = o.pick[1];
  row0 = o.row0[r];
  qo = o.qo[r];
  kv = o.kv[r];
  __syncthreads();   // the ordering's LDS is ring space again
  return r;
}

template <int RT, int D, int KDT, int MODE, int OCC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, OCC)))
sdv_attn_waves_kernel(AttnArgs a, DenseSource ds, SparseSource ss) {
  __shared__ WavesLds<RT, D, KDT, MODE> sh;
  // Grid x = (request, KV head), y = split, so consecutive workgroups (dealt round-robin
  // to the XCDs) are different (request, head) pairs of one split; the request index is
  // rotated by the split, so a request's splits alternate between XCDs.
  const int Hkv = a.num_kv_heads;
  const int split = blockIdx.y;
  const int h = blockIdx.x % Hkv;
  const int pos = static_cast<int>((blockIdx.x / Hkv + split) % static_cast<uint32_t>(a.B));
  int r, row0, qo, kv;
  if constexpr (is_sparse(MODE)) {
    static_assert(sizeof(OrderLds) <= sizeof(sh.ring), "the ordering fits the ring");
    if (a.order_by_work) {
      r = request_by_work(*reinterpret_cast<OrderLds*>(sh.ring), a, ss, pos, row0, qo, kv);
    } else {
      r = pos;
      row0 = a.qo_indptr[r];
      qo = a.qo_indptr[r + 1] - row0;
      kv = a.kv_len[r];
    }
  } else {
    r = pos;
    row0 = a.qo_indptr[r];
    qo = a.qo_indptr[r + 1] - row0;
    kv = a.kv_len[r];
  }
  const int64_t kv_cap = MODE == kSrcView ? static_cast<int64_t>(ds.max_sub_pages) * kSub
                                           : static_cast<int64_t>(ss.max_pages) * kPage;
  const bool bad_len = qo < 1 || qo > a.max_qo_len || kv < qo || row0 < 0 ||
                       static_cast<int64_t>(row0) + qo > static_cast<int64_t>(a.B) * a.max_qo_len;
  const bool bad_cap = !bad_len && kv > kv_cap;
  if (bad_len || bad_cap) {
    if (threadIdx.x == 0 && split == 0 && h == 0)
      set_err(a.dev_err, bad_len ? SDV_DEVERR_QO_LEN : SDV_DEVERR_KV_CAPACITY);
    return;
  }
  // The split's block list, staged in LDS, read back one block ahead of use.
  BlockList<MODE, D, KDT> bl;
  bl.stage(sh.ul, &sh.chunk, a, ds, ss, r, h, split, row0, qo, kv);
  waves_attend<RT, D, KDT, MODE>(sh, a, ds, ss, bl, r, h, row0, qo, kv,
                                 a.num_splits > 1 ? split : -1);
}

// Dense persistent variant: equal ranges of 32-token blocks per workgroup across all
// (request, KV head) pairs (persistent_walk), each piece attended as above.
template <int RT, int D, int KDT, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
sdv_attn_waves_persist_kernel(AttnArgs a, DenseSource ds, SparseSource ss) {
  static_assert(!is_sparse(MODE), "dense sources only");
  __shared__ WavesLds<RT, D, KDT, MODE> sh;
  __shared__ PersistLds pl;
  persistent_walk<MODE>(pl, a, ds, ss,
                        [&](int r, int h, int row0, int qo, int kv, int first, int n, int slot) {
                          BlockList<MODE, D, KDT> bl;
                          bl.stage_range(sh.ul, a, ds, ss, r, first, n);
                          waves_attend<RT, D, KDT, MODE>(sh, a, ds, ss, bl, r, h, row0, qo, kv, slot);
                        });
}

template <int RT, int D, int KDT, int MODE>
hipError_t launch_t(const AttnArgs& a, const DenseSource& ds, const SparseSource& ss,
                    hipStream_t s) {
  constexpr int OCC = waves_occupancy<RT, D, KDT, MODE>();
  static const int per_cu = resident_per_cu(sdv_attn_waves_kernel<RT, D, KDT, MODE, OCC>);
  AttnArgs args = a;
  args.target_wgs = per_cu * device_cu_count();
  // Longest-first order where the grid runs in several generations (from the shapes only).
  args.order_by_work = is_sparse(MODE) && a.B <= kOrderMaxRequests &&
                       static_cast<int64_t>(a.num_kv_heads) * a.B * a.num_splits > args.target_wgs;
  dim3 grid(a.num_kv_heads * a.B, a.num_splits);
  hipLaunchKernelGGL((sdv_attn_waves_kernel<RT, D, KDT, MODE, OCC>), grid, dim3(256), 0, s, args,
                     ds, ss);
  return hipGetLastError();
}

template <int RT, int D, int KDT, int MODE>
hipError_t launch_persist_t(const AttnArgs& a, const DenseSource& ds, const SparseSource& ss,
                            int64_t cap_blocks, hipStream_t s) {
  static const int per_cu = resident_per_cu(sdv_attn_waves_persist_kernel<RT, D, KDT, MODE>);
  AttnArgs args = a;
  args.target_wgs = per_cu * device_cu_count();
  // enough workgroups for ranges of kMaxDenseBlocks when the balanced length is longer
  const int64_t need = (static_cast<int64_t>(a.B) * a.num_kv_heads * cap_blocks + kMaxDenseBlocks - 1) /
                       kMaxDenseBlocks;
  const int64_t wgs = std::max<int64_t>(args.target_wgs, need);
  hipLaunchKernelGGL((sdv_attn_waves_persist_kernel<RT, D, KDT, MODE>), dim3(static_cast<uint32_t>(wgs)),
                     dim3(256), 0, s, args, ds, ss);
  return hipGetLastError();
}

template <int MODE, bool PERSIST>
hipError_t dispatch(const AttnArgs& a, const DenseSource& ds, const SparseSource& ss,
                    int64_t cap_blocks, hipStream_t s) {
  const int rows = a.max_qo_len * (a.num_q_heads / a.num_kv_heads);
  const int rt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
#define SDV_WAVES_CASE(RTV, DV, KDTV)                                                  \
  if (rt == RTV && a.head_dim == DV && a.kv_dt == KDTV) {                              \
    if constexpr (PERSIST) return launch_persist_t<RTV, DV, KDTV, MODE>(a, ds, ss, cap_blocks, s); \
    else return launch_t<RTV, DV, KDTV, MODE>(a, ds, ss, s);                           \
  }
  SDV_WAVES_CASE(1, 128, SDV_BF16)
  SDV_WAVES_CASE(2, 128, SDV_BF16)
  SDV_WAVES_CASE(4, 128, SDV_BF16)
  SDV_WAVES_CASE(1, 64, SDV_BF16)
  SDV_WAVES_CASE(2, 64, SDV_BF16)
  SDV_WAVES_CASE(4, 64, SDV_BF16)
  SDV_WAVES_CASE(1, 128, SDV_FP8_E4M3)
  SDV_WAVES_CASE(2, 128, SDV_FP8_E4M3)
  SDV_WAVES_CASE(4, 128, SDV_FP8_E4M3)
  SDV_WAVES_CASE(1, 64, SDV_FP8_E4M3)
  SDV_WAVES_CASE(2, 64, SDV_FP8_E4M3)
  SDV_WAVES_CASE(4, 64, SDV_FP8_E4M3)
#undef SDV_WAVES_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_dense_waves(const AttnArgs& a, const DenseSource& src, hipStream_t s) {
  return dispatch<kSrcView, false>(a, src, SparseSource{}, 0, s);
}

hipError_t launch_attn_sparse_waves(const AttnArgs& a, const SparseSource& src, hipStream_t s) {
  if (src.scores)
    return select_wide(src) ? dispatch<kSrcSparseSelectWide, false>(a, DenseSource{}, src, 0, s)
                            : dispatch<kSrcSparseSelect, false>(a, DenseSource{}, src, 0, s);
  return dispatch<kSrcSparse, false>(a, DenseSource{}, src, 0, s);
}

hipError_t launch_attn_paged_waves(const AttnArgs& a, const SparseSource& src, hipStream_t s) {
  return dispatch<kSrcPaged, false>(a, DenseSource{}, src, 0, s);
}

bool persist_supported(const AttnArgs& a, int64_t cap_blocks) {
  if (a.num_splits < 2 || a.B > kPersistMaxRequests || cap_blocks < 1) return false;
  if ((cap_blocks + a.num_splits - 2) / (a.num_splits - 1) > kMaxDenseBlocks) return false;
  // every flattened block index and every split slot's row index fits in 32 bits
  return static_cast<int64_t>(a.B) * a.num_kv_heads * cap_blocks <= INT32_MAX;
}

hipError_t launch_attn_dense_persist(const AttnArgs& a, const DenseSource& src, hipStream_t s) {
  return dispatch<kSrcView, true>(a, src, SparseSource{}, src.max_sub_pages, s);
}

hipError_t launch_attn_paged_persist(const AttnArgs& a, const SparseSource& src, hipStream_t s) {
  return dispatch<kSrcPaged, true>(a, DenseSource{}, src, 4ll * src.max_pages, s);
}

}  // namespace sdv
