// Verify attention on the CDNA4 matrix cores with an LDS block ring (bf16 queries;
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
//   * One workgroup (4 waves) per (request, KV head, split).  Its query rows are the
//     G x qo (token, head) pairs, row = t * G + g, in RT tiles of 16 (RT = 1, 2, 4).
//     Wave w owns row tile w % RT and the output channel part w / RT of 4 / RT parts,
//     so every wave works on every 32-token block of the split: with 64 rows the waves
//     split the rows, with 16 rows they split the value product's output channels
//     (and compute the same scores).
//   * Each 32-token K/V block is copied once from HBM into an LDS ring by the
//     asynchronous global->LDS loads (global_load_lds_dwordx4): each wave instruction
//     reads one contiguous KiB of K or V.  STAGES - 1 blocks are in flight while one is
//     computed; no registers hold in-flight data.  The 16-byte chunks of a row land
//     XOR-swizzled by the row number, so the MFMA operand reads (16 rows, same column)
//     and the value reads (one row, all columns) are free of LDS bank conflicts.
//   * Scores are computed transposed, S^T = K Q^T (K the A operand, Q^T the B operand
//     held in registers); lane l then holds query row l % 16 for tokens 4(l/16)..+3 of
//     each 16-token tile — the B-operand layout of O^T = V^T P^T — so the probabilities
//     feed the value product with no data exchange, and each query row's online-softmax
//     rescale is a per-lane multiply.  Channels within a 32-channel step are permuted
//     (lane group q takes channels q*d/4 .. q*d/4 + d/4 - 1 across the steps), the same
//     for K and Q, which leaves the dot products unchanged.
//   * Output goes through LDS to coalesced stores: the final rows, or a normalised
//     partial with its log-sum-exp for the split-KV combine.
#include "mfma_attn.h"
#include "sparse_union.h"

namespace sdv {
namespace {

// Ring depth (blocks): ST - 1 blocks are in flight while one is computed, so a deeper
// ring hides more memory latency per workgroup, at the price of LDS and so of
// workgroups per CU (measured: 6 and 8 slots at one workgroup per CU are slower than 4
// at two).
constexpr int kRingStages = 4;

// LDS of the ring kernels: the block ring (after the last block the same bytes stage
// the output rows), the rows' maxima and sums, and the staged block list.
template <int RT, int D, int KDT, int MODE, int ST>
struct RingLds {
  using Gm = Geo<D, KDT>;
  static constexpr int ROWS = RT * 16;
  static constexpr int OPAD = D + 4;
  static constexpr int RING = ST * Gm::BLOCK;
  static constexpr int OUTB = ROWS * OPAD * 4;
  __attribute__((aligned(16))) char ring[RING > OUTB ? RING : OUTB];
  float L[ROWS];
  float M[ROWS];
  typename BlockList<MODE, D, KDT>::Lds ul;
  int chunk;
};

// Attention of the G x qo query rows of (request r, KV head h) over the staged block
// range `bl` (metadata in sh.ul), written as the final rows (out_slot < 0) or as the
// normalised partial and log-sum-exp of split slot out_slot.  All 256 threads call; LDS
// is free again only after a barrier that follows the call.
template <int RT, int D, int KDT, int MODE, int ST>
__device__ __forceinline__ void ring_attend(RingLds<RT, D, KDT, MODE, ST>& sh, const AttnArgs& a,
                                            const DenseSource& ds, const SparseSource& ss,
                                            const BlockList<MODE, D, KDT>& bl, int r, int h,
                                            int row0, int qo, int kv, int out_slot) {
  using Gm = Geo<D, KDT>;
  using BL = BlockList<MODE, D, KDT>;
  constexpr int STEPS = Gm::STEPS;
  constexpr int NT = Gm::NT;
  constexpr int NCP = 4 / RT;          // output-channel parts
  constexpr int NTW = NT / NCP;        // output tiles per wave
  constexpr int OPAD = D + 4;
  constexpr int kStages = ST;
  static_assert(NTW >= 1, "tiles per wave");
  float (*o_lds)[OPAD] = reinterpret_cast<float (*)[OPAD]>(sh.ring);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int i = lane & 15;
  const int q = lane >> 4;
  const int rt = wave % RT;
  const int cp = wave / RT;
  const int n0 = cp * NTW;
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int nrows = qo * G;

  // This wave's query row (lane i of row tile rt), its token and its ladder bound.
  const int row = rt * 16 + i;
  const bool row_live = row < nrows;
  const int t_row = row_live ? row / G : 0;
  const int g_row = row_live ? row - t_row * G : 0;
  const int bound_row = row_live ? kv - qo + t_row + 1 : 0;
  const float qk_scale = a.softmax_scale * a.k_scale * kLog2e;

  const int nblk = bl.nblk;

  // Metadata of block b as stored in LDS (wave-uniform values, still in vector registers).
  // It is fetched one block ahead of its use, so the read's latency hides under compute.
  auto fetch = [&](int b) { return bl.fetch(sh.ul, b); };
  auto resolve = [&](const typename BL::Raw& m, int b, uint64_t& kbase, uint64_t& vbase, int& pos0,
                     int& mask) { bl.resolve(m, b, h, Hkv, ds, ss, kbase, vbase, pos0, mask); };

  BlockCopier<D, KDT> copier;
  copier.init(__builtin_amdgcn_readfirstlane(wave), lane);
  const uint32_t ring_lds = lds_address(sh.ring);
  // Blocks wholly inside every row's ladder bound and chosen by every token need no
  // masking: the common case, tested once per block for the whole workgroup.
  const int all_tokens = qo >= 32 ? ~0 : (1 << qo) - 1;
  const int first_bound = kv - qo + 1;

  f32x4 o[NTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // First position and selecting tokens of the block each ring slot holds.
  int slot_pos[kStages], slot_mask[kStages];
#pragma unroll
  for (int j = 0; j < kStages; ++j) slot_pos[j] = slot_mask[j] = 0;

  // Prologue: blocks 0 .. kStages - 2 in flight.
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j) {
    if (j < nblk) {
      uint64_t kb, vb;
      resolve(fetch(j), j, kb, vb, slot_pos[j], slot_mask[j]);
      copier.issue(kb, vb, ring_lds + j * Gm::BLOCK);
    }
  }
  typename BL::Raw next{0, 0, 0};
  if (kStages - 1 < nblk) next = fetch(kStages - 1);

  // The query rows load while the first blocks' copies are in flight; one wait then
  // covers both, so no wait inside the block loop has to account for Q (the compiler,
  // which does not see the copies, would otherwise wait for everything in flight there).
  bf16x8 qb[STEPS];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(row0 + t_row) * a.num_q_heads + h * G + g_row) * D +
                      q * (D / 4)) * 2;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const uint4 w = row_live ? *reinterpret_cast<const uint4*>(qp + Gm::step_unit(q, s) * 16)
                               : make_uint4(0, 0, 0, 0);
      qb[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // Block b lives in slot b % kStages; the loop runs kStages blocks per trip so that every
  // slot offset and slot register index is a compile-time constant.
  auto step = [&](auto slot_c, int b) {
    constexpr int u = decltype(slot_c)::value;
    constexpr int un = (u + kStages - 1) % kStages;   // slot of block b - 1 = of b + kStages - 1
    // This wave's LDS reads of block b - 1 and the metadata fetch are complete and its
    // copies of block b have landed; the barrier extends both facts to every wave.
    wait_lgkmcnt0();
    wait_blocks<Gm::LPT, kStages - 2>(min(nblk - 1 - b, kStages - 2));
    ring_barrier();

    // All of this wave's reads of the block first, so their latency runs under the copy
    // issue below and under the score products.
    const char* kb = sh.ring + u * Gm::BLOCK;
    const char* vb = kb + Gm::HALF;
    bf16x8 kop[2][STEPS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < STEPS; ++s) kop[tt][s] = k_operand<D, KDT>(kb, tt, s, i, q);
    uint32_t vraw[8][4];
    v_runs<D, KDT, NTW>(vb, i, q, n0, vraw);

    const int bn = b + kStages - 1;
    if (bn < nblk) {
      uint64_t kbn, vbn;
      resolve(next, bn, kbn, vbn, slot_pos[un], slot_mask[un]);
      copier.issue(kbn, vbn, ring_lds + un * Gm::BLOCK);
      if (bn + 1 < nblk) next = fetch(bn + 1);
    }

    const int pos0 = slot_pos[u];
    const int mask = slot_mask[u];
    const bool inside = pos0 + kSub <= first_bound && (mask & all_tokens) == all_tokens;

    // scores S^T for this wave's row tile (unscaled)
    f32x4 sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < STEPS; ++s) sacc[tt] = mfma16(kop[tt][s], qb[s], sacc[tt]);
    }
    float mx = -INFINITY;
    if (inside) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[tt][e]);
    } else {
      const int bnd = ((mask >> t_row) & 1) ? bound_row : 0;
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
    // The scale is positive, so scaling the maximum equals the maximum of the scaled
    // scores.  The row's reference maximum moves only when a score exceeds it by more
    // than 2^8 (probabilities then stay <= 256); l and O always share the reference, so
    // the normalised result is unchanged and most blocks skip the rescale.  A row's
    // maximum can pass the threshold only if one of its four lanes' partial maxima does,
    // so the cross-lane reduction runs only when some lane of the wave votes for it.
    const float mx_scaled = mx * qk_scale;
    if (__any(mx_scaled > m_run + kRescaleLog2)) {
      float mr = fmaxf(mx_scaled, __shfl_xor(mx_scaled, 16, kWave));
      mr = fmaxf(mr, __shfl_xor(mr, 32, kWave));
      if (mr > m_run + kRescaleLog2) {
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mr);
        l_run *= alpha;
#pragma unroll
        for (int n = 0; n < NTW; ++n) o[n] *= alpha;
        m_run = mr;
      }
    }
    // Masked scores are -inf and give 0; a row with no live score yet keeps m = -inf and
    // has only masked scores here.
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float p[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[0][e], qk_scale, -m_use));
      p[e + 4] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[1][e], qk_scale, -m_use));
    }
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ls += p[e];
    l_run += ls;
    const bf16x8 pb = __builtin_bit_cast(
        bf16x8, make_uint4(pack2_bf16(p[0], p[1]), pack2_bf16(p[2], p[3]), pack2_bf16(p[4], p[5]),
                           pack2_bf16(p[6], p[7])));
    // value product for this wave's output tiles; positions past kv_len read as 0 (stale
    // storage must not reach P * V, even times a zero probability)
    if (pos0 + kSub > kv) v_zero_tail(q, pos0, kv, vraw);
#pragma unroll
    for (int n = 0; n < NTW; ++n) o[n] = mfma16(v_operand<KDT>(vraw, n), pb, o[n]);
  };

  for (int b0 = 0; b0 < nblk; b0 += kStages) {
    static_for<kStages>([&](auto slot_c) {
      const int b = b0 + decltype(slot_c)::value;
      if (b < nblk) step(slot_c, b);
    });
  }
  wait_vmcnt<0>();
  __syncthreads();

  // ---- normalise and write (waves of one row tile hold identical m, l) ----
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  if (cp == 0 && q == 0) {
    sh.L[row] = l_run;
    sh.M[row] = m_run;
  }
#pragma unroll
  for (int n = 0; n < NTW; ++n)
#pragma unroll
    for (int e = 0; e < 4; ++e) o_lds[row][NT * (4 * q + e) + n0 + n] = o[n][e];
  __syncthreads();

  const int64_t rows_cap = static_cast<int64_t>(a.B) * a.max_qo_len;
  for (int item = tid; item < nrows * (D / 8); item += 256) {
    const int orow = item / (D / 8);
    const int c0 = (item - orow * (D / 8)) * 8;
    const int t = orow / G;
    const int g = orow - t * G;
    const int hq = h * G + g;
    const int64_t qrow = row0 + t;
    const float L = sh.L[orow];
    const float inv = L > 0.f ? a.v_scale / L : 0.f;
    float v8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v8[e] = o_lds[orow][c0 + e] * inv;
    if (out_slot < 0) {
      const int64_t idx = (qrow * a.num_q_heads + hq) * D + c0;
      if (a.out_dt == SDV_BF16) {
        const uint4 w = make_uint4(pack2_bf16(v8[0], v8[1]), pack2_bf16(v8[2], v8[3]),
                                   pack2_bf16(v8[4], v8[5]), pack2_bf16(v8[6], v8[7]));
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + idx) = w;
      } else {
        float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + idx);
        dst[0] = make_float4(v8[0], v8[1], v8[2], v8[3]);
        dst[1] = make_float4(v8[4], v8[5], v8[6], v8[7]);
      }
    } else {
      // A row with no live position (an empty split) leaves its partial output unwritten:
      // the combine skips rows whose log-sum-exp is -inf.
      const int64_t unit = (static_cast<int64_t>(out_slot) * rows_cap + qrow) * a.num_q_heads + hq;
      if (L > 0.f) {
        float4* dst = reinterpret_cast<float4*>(a.part_o + unit * D + c0);
        dst[0] = make_float4(v8[0], v8[1], v8[2], v8[3]);
        dst[1] = make_float4(v8[4], v8[5], v8[6], v8[7]);
      }
      if (c0 == 0)
        a.part_lse[unit] = L > 0.f ? (sh.M[orow] + __log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

template <int RT, int D, int KDT, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8)))
sdv_attn_stream_kernel(AttnArgs a, DenseSource ds, SparseSource ss) {
  __shared__ RingLds<RT, D, KDT, MODE, kRingStages> sh;
  // Grid x = (request, KV head), y = split: consecutive workgroups, which the hardware
  // deals round-robin to the eight XCDs, are different (request, head) pairs of the same
  // split, so long and short requests spread evenly over the XCDs, and the high splits
  // (empty for short requests) are dispatched last.  The request index is rotated by the
  // split, so that a request's splits alternate between XCDs instead of all landing on the
  // XCDs its unrotated position picks (with four KV heads, one half of them): 78 -> 76 us
  // on 32 requests of U[1024, 8192] bf16 tokens at 4 splits, 92 -> 85 us at 8.  Dense
  // calls with splits number their pieces by dense_compact_piece instead (77 -> 73-75 us
  // on the same requests at 6 splits).
  const int Hkv = a.num_kv_heads;
  int split = blockIdx.y;
  int h = blockIdx.x % Hkv;
  int r = static_cast<int>((blockIdx.x / Hkv + split) % static_cast<uint32_t>(a.B));
  const int64_t kv_cap = MODE == kSrcView ? static_cast<int64_t>(ds.max_sub_pages) * kSub
                                           : static_cast<int64_t>(ss.max_pages) * kPage;
  // Dense split-KV: grid positions take the pieces sized to the requests instead (the
  // ring is free before the first copy).
  DensePiece pc{};
  int row0, qo, kv;
  bool compact = false;
  if constexpr (!is_sparse(MODE)) {
    if (a.dense_compact) {
      const int cap = MODE == kSrcView ? ds.max_sub_pages : 4 * ss.max_pages;
      if (!dense_compact_piece(a, cap, reinterpret_cast<int*>(sh.ring), pc)) return;
      compact = true;
      r = pc.r;
      h = pc.h;
      split = pc.j;
    }
  }
  if (compact) {
    row0 = pc.row0;
    qo = pc.qo;
    kv = pc.kv;
  } else {
    row0 = a.qo_indptr[r];
    qo = a.qo_indptr[r + 1] - row0;
    kv = a.kv_len[r];
  }
  const bool bad_len = qo < 1 || qo > a.max_qo_len || kv < qo || row0 < 0 ||
                       static_cast<int64_t>(row0) + qo > static_cast<int64_t>(a.B) * a.max_qo_len;
  const bool bad_cap = !bad_len && kv > kv_cap;
  if (bad_len || bad_cap) {
    if (threadIdx.x == 0 && split == 0 && h == 0)
      set_err(a.dev_err, bad_len ? SDV_DEVERR_QO_LEN : SDV_DEVERR_KV_CAPACITY);
    return;
  }
  BlockList<MODE, D, KDT> bl;
  if constexpr (!is_sparse(MODE)) {
    if (compact) {
      // the pair's run 0 marks the partial slots past its last run empty for the combine
      if (split == 0) {
        const int G = a.num_q_heads / Hkv;
        const int64_t rows_cap = static_cast<int64_t>(a.B) * a.max_qo_len;
        const int n_fill = (a.num_splits - pc.k) * qo * G;
        for (int e = threadIdx.x; e < n_fill; e += blockDim.x) {
          const int s = pc.k + e / (qo * G);
          const int t = (e / G) % qo;
          const int g = e % G;
          a.part_lse[(s * rows_cap + row0 + t) * a.num_q_heads + h * G + g] = -INFINITY;
        }
      }
      bl.stage_range(sh.ul, a, ds, ss, r, pc.first, pc.n);
      ring_attend<RT, D, KDT, MODE, kRingStages>(sh, a, ds, ss, bl, r, h, row0, qo, kv, split);
      return;
    }
  }
  bl.stage(sh.ul, &sh.chunk, a, ds, ss, r, h, split, row0, qo, kv);
  ring_attend<RT, D, KDT, MODE, kRingStages>(sh, a, ds, ss, bl, r, h, row0, qo, kv,
                                             a.num_splits > 1 ? split : -1);
}

template <int RT, int D, int KDT, int MODE>
hipError_t launch_t(const AttnArgs& a, const DenseSource& ds, const SparseSource& ss,
                    hipStream_t s) {
  static const int per_cu = resident_per_cu(sdv_attn_stream_kernel<RT, D, KDT, MODE>);
  AttnArgs args = a;
  args.target_wgs = per_cu * device_cu_count();
  args.dense_compact = !is_sparse(MODE) && a.num_splits > 1 && a.B <= kCompactMaxRequests;
  dim3 grid(a.num_kv_heads * a.B, a.num_splits);
  hipLaunchKernelGGL((sdv_attn_stream_kernel<RT, D, KDT, MODE>), grid, dim3(256), 0, s, args, ds, ss);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(const AttnArgs& a, const DenseSource& ds, const SparseSource& ss,
                    hipStream_t s) {
  const int rows = a.max_qo_len * (a.num_q_heads / a.num_kv_heads);
  const int rt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
#define SDV_STREAM_CASE(RTV, DV, KDTV)                                                 \
  if (rt == RTV && a.head_dim == DV && a.kv_dt == KDTV)                                \
    return launch_t<RTV, DV, KDTV, MODE>(a, ds, ss, s);
  SDV_STREAM_CASE(1, 128, SDV_BF16)
  SDV_STREAM_CASE(2, 128, SDV_BF16)
  SDV_STREAM_CASE(4, 128, SDV_BF16)
  SDV_STREAM_CASE(1, 64, SDV_BF16)
  SDV_STREAM_CASE(2, 64, SDV_BF16)
  SDV_STREAM_CASE(4, 64, SDV_BF16)
  SDV_STREAM_CASE(1, 128, SDV_FP8_E4M3)
  SDV_STREAM_CASE(2, 128, SDV_FP8_E4M3)
  SDV_STREAM_CASE(4, 128, SDV_FP8_E4M3)
  SDV_STREAM_CASE(1, 64, SDV_FP8_E4M3)
  SDV_STREAM_CASE(2, 64, SDV_FP8_E4M3)
  SDV_STREAM_CASE(4, 64, SDV_FP8_E4M3)
#undef SDV_STREAM_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_dense_stream(const AttnArgs& a, const DenseSource& src, hipStream_t s) {
  return dispatch<kSrcView>(a, src, SparseSource{}, s);
}

hipError_t launch_attn_sparse_stream(const AttnArgs& a, const SparseSource& src, hipStream_t s) {
  if (src.scores)
    return select_wide(src) ? dispatch<kSrcSparseSelectWide>(a, DenseSource{}, src, s)
                            : dispatch<kSrcSparseSelect>(a, DenseSource{}, src, s);
  return dispatch<kSrcSparse>(a, DenseSource{}, src, s);
}

hipError_t launch_attn_paged_stream(const AttnArgs& a, const SparseSource& src, hipStream_t s) {
  return dispatch<kSrcPaged>(a, DenseSource{}, src, s);
}

}  // namespace sdv
