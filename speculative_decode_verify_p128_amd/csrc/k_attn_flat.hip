// Dense verify attention under the persistent split-KV partition, with one block
// pipeline per workgroup that runs straight through the boundaries between (request,
// KV head) pieces (bf16 queries; bf16 or fp8 K/V; dense sources only).
//
// What is computed is the same as in the LDS-ring kernel: token t of request r, query
// head hq of KV head h attends the positions j < bound(r,t) = kv_len - qo_len + t + 1
// ("[TRTLLM-14093][feat] Eagle3 for M3 MSA path + CUDA graphs compatibility", MSA
// verify commit), the keys coming through the P32 sub-page view of the draft layer's
// P128 pages ("[None][perf] Default Minimax-m3 to unified draft-target kv manager ...",
// Description and item 2 Grouped-HND) or from head-major P128 pages.
//
// The (request, KV head) pairs, request-major, laid end to end form one list of 32-token
// blocks; workgroup g takes blocks [g L, (g + 1) L) of it (persistent_prefix), which
// may hold the tail of one pair, whole short pairs and the head of another.  With kv_len
// spread over a range, per-(pair, split) workgroups leave the longest pairs' workgroups
// running alone at the end; here every CU streams the same number of blocks.  A piece
// of a pair becomes the partial of split slot (g - first workgroup of the pair), merged
// by the ordinary combine.
//
// Restarting the ring for every piece costs a query load, a block-list load, the ring's
// fill and an output pass through LDS, each a memory round trip (measured slower than the
// per-split grid).  This kernel plans the whole range first instead: the pieces, their
// requests' lengths and every block's page index go to LDS, and then the ring runs over
// the range without a break.  A piece's query rows are copied into LDS by the same
// asynchronous copies as the K/V blocks, issued with the copies of the piece's first
// block (one query buffer per ring slot), so they have landed when that block is
// computed; a finished piece is normalised and written from registers, each lane
// storing the runs of output channels it holds.
#include "mfma_attn.h"

namespace sdv {
namespace {

constexpr int kFlatMaxPieces = 64; // pieces planned at once (more: the range is cut)

struct FlatPiece {
  int r, h, row0, qo, kv;
  int first;   // the piece's first block within its pair
  int start;   // its first block within the planned run
  int slot;    // split slot of the partial
  int nb;      // blocks of its pair
};

// LDS bytes of the flat kernel with st ring slots.  The request prefix shares the ring's
// bytes: it is read only while a range is planned, before the ring runs.
template <int RT, int D, int KDT>
constexpr int flat_lds_bytes(int st) {
  return st * Geo<D, KDT>::BLOCK + st * RT * 16 * D * 2 + kMaxDenseBlocks * 4 +
         (kFlatMaxPieces + 1) * static_cast<int>(sizeof(FlatPiece));
}

// Ring slots: four (three blocks in flight while one is computed), or three where that
// lets two workgroups share a CU (80 KiB of LDS each) and four do not.  Only row tiles of
// up to 32 rows leave the registers of two waves per SIMD; 64-row tiles keep four slots.
template <int RT, int D, int KDT>
constexpr int flat_stages() {
  constexpr int kTwoPerCu = 80 * 1024;
  return RT > 2 || flat_lds_bytes<RT, D, KDT>(4) <= kTwoPerCu ? 4
         : flat_lds_bytes<RT, D, KDT>(3) <= kTwoPerCu ? 3 : 4;
}

template <int RT, int D, int KDT>
struct FlatLds {
  using Gm = Geo<D, KDT>;
  static constexpr int ST = flat_stages<RT, D, KDT>();
  static constexpr int ROWS = RT * 16;
  static constexpr int QBYTES = ROWS * D * 2;   // one piece's query rows, bf16 [row][D]
  static_assert(sizeof(PersistLds) <= ST * Gm::BLOCK, "the request prefix fits the ring");
  union {
    __attribute__((aligned(16))) char ring[ST * Gm::BLOCK];
    PersistLds pl;                          // while a range is planned
  };
  __attribute__((aligned(16))) char qbuf[ST * QBYTES];
  int x[kMaxDenseBlocks];                   // page index of each planned block, -1 invalid
  FlatPiece piece[kFlatMaxPieces + 1];      // + sentinel: piece[n].start = planned blocks
};

template <int RT, int D, int KDT, int MODE>
__device__ __forceinline__ void flat_attend(FlatLds<RT, D, KDT>& sh, const AttnArgs& a,
                                            const DenseSource& ds, const SparseSource& ss,
                                            int nblk) {
  using Gm = Geo<D, KDT>;
  using LdsT = FlatLds<RT, D, KDT>;
  constexpr int STEPS = Gm::STEPS;
  constexpr int NT = Gm::NT;
  constexpr int NCP = 4 / RT;          // output-channel parts
  constexpr int NTW = NT / NCP;        // output tiles per wave
  constexpr int kStages = LdsT::ST;
  constexpr int QI = LdsT::QBYTES / 1024;           // 1 KiB copy instructions per query tile
  constexpr int QPW = (QI + 3) / 4;                 // per wave
  static_assert(NTW >= 1 && QI >= 1, "tiles per wave");
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i = lane & 15;
  const int q = lane >> 4;
  const int rt = wave % RT;
  const int cp = wave / RT;
  const int n0 = cp * NTW;
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int row = rt * 16 + i;          // this lane's query row within a piece
  const float qk_scale = a.softmax_scale * a.k_scale * kLog2e;
  const int64_t rows_cap = static_cast<int64_t>(a.B) * a.max_qo_len;

  BlockCopier<D, KDT> copier;
  copier.init(wave, lane);
  const uint32_t ring_lds = lds_address(sh.ring);
  const uint32_t qbuf_lds = lds_address(sh.qbuf);

  // ---- issue side: block jb of the planned run into ring slot u ----
  // The fields of the piece being issued stay in scalar registers and are reloaded from
  // LDS only when a piece begins; each block's page index is read one block ahead, so no
  // LDS latency sits between two blocks' copies.
  int ki = 0;
  int i_start = 0, i_end = 0, i_h = 0, i_first = 0, i_kv = 0, i_row0 = 0, i_qo = 1;
  auto load_issue_piece = [&](int k) {
    i_start = __builtin_amdgcn_readfirstlane(sh.piece[k].start);
    i_end = __builtin_amdgcn_readfirstlane(sh.piece[k + 1].start);
    i_h = __builtin_amdgcn_readfirstlane(sh.piece[k].h);
    i_first = __builtin_amdgcn_readfirstlane(sh.piece[k].first);
    i_kv = __builtin_amdgcn_readfirstlane(sh.piece[k].kv);
    i_row0 = __builtin_amdgcn_readfirstlane(sh.piece[k].row0);
    i_qo = __builtin_amdgcn_readfirstlane(sh.piece[k].qo);
  };
  load_issue_piece(0);
  int x_next = sh.x[0];
  int slot_pos[kStages], slot_mask[kStages], slot_kv[kStages];
#pragma unroll
  for (int u = 0; u < kStages; ++u) slot_pos[u] = slot_mask[u] = slot_kv[u] = 0;

  // This wave's share of the issued piece's query rows into query buffer u (rows past
  // the piece's rows repeat its last row: in bounds, and never read as a live row).
  auto issue_q = [&](int u) {
    const int h = i_h;
    const int row0 = i_row0;
    const int nrows = i_qo * G;
#pragma unroll
    for (int n = 0; n < QPW; ++n) {
      const int ins = wave * QPW + n;
      if (ins < QI) {
        const int byte = ins * 1024 + lane * 16;
        const int rho = min(byte / (D * 2), nrows - 1);
        const int c = byte % (D * 2);
        const int t = rho / G;
        const uint64_t addr = reinterpret_cast<uint64_t>(a.q) +
            static_cast<uint64_t>(((static_cast<int64_t>(row0 + t) * a.num_q_heads + h * G +
                                    (rho - t * G)) * D) * 2 + c);
        const uint32_t m0 = qbuf_lds + u * LdsT::QBYTES + ins * 1024;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(m0), "v"(addr)
                     : "memory", "m0");
#pragma clang diagnostic pop
      }
    }
  };

  auto issue = [&](auto slot_c, int jb) {
    constexpr int u = decltype(slot_c)::value;
    if (jb == i_end) load_issue_piece(++ki);   // pieces hold at least one block
    const int h = i_h;
    const int pb = i_first + (jb - i_start);
    if (jb == i_start) issue_q(u);
    int64_t x = __builtin_amdgcn_readfirstlane(x_next);
    if (jb + 1 < nblk) x_next = sh.x[jb + 1];
    slot_mask[u] = x < 0 ? 0 : ~0;
    x = x < 0 ? 0 : x;
    slot_pos[u] = pb * kSub;
    slot_kv[u] = i_kv;
    uint64_t kbase, vbase;
    if constexpr (MODE == kSrcView) {
      kbase = reinterpret_cast<uint64_t>(ds.root) +
              static_cast<uint64_t>((x * Hkv + h) * kSub * D * Gm::EB);
      vbase = reinterpret_cast<uint64_t>(ds.root) +
              static_cast<uint64_t>(((x + 4) * Hkv + h) * kSub * D * Gm::EB);
    } else {
      const uint64_t off = static_cast<uint64_t>(
          (x * ss.page_stride + (static_cast<int64_t>(h) * kPage + (pb & 3) * kSub) * D) * Gm::EB);
      kbase = reinterpret_cast<uint64_t>(ss.k) + off;
      vbase = reinterpret_cast<uint64_t>(ss.v) + off;
    }
    copier.issue(kbase, vbase, ring_lds + u * Gm::BLOCK);
  };

  // ---- compute side: the piece in progress ----
  int kc = -1;
  int c_next = 0;                       // first block of the next piece
  int h_c = 0, row0_c = 0, slot_c = 0, qo_c = 1;
  bool row_live = false;
  int t_row = 0, bound_row = 0, first_bound = 0, all_tokens = 0;
  bf16x8 qb[STEPS];
  f32x4 o[NTW];
  float m_run = -INFINITY, l_run = 0.f;

  // Normalise a finished piece and write its partial and log-sum-exp (a row with no live
  // position leaves its partial unwritten and lse = -inf, which the combine skips).  Every
  // lane calls: the row sum is reduced across the lane groups first.
  auto store_partial = [&](const f32x4 (&od)[NTW], float m, float lsum, int slot, int row0,
                           int h, int qo) {
    float l = lsum + __shfl_xor(lsum, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (row < qo * G) {
      const int t = row / G;
      const int64_t unit = (static_cast<int64_t>(slot) * rows_cap + row0 + t) * a.num_q_heads +
                           h * G + (row - t * G);
      if (l > 0.f) {
        const float inv = a.v_scale / l;
        float* dst = a.part_o + unit * D;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float* d0 = dst + NT * (4 * q + e) + n0;
          if constexpr (NTW % 4 == 0) {
#pragma unroll
            for (int n = 0; n < NTW; n += 4)
              *reinterpret_cast<float4*>(d0 + n) = make_float4(od[n][e] * inv, od[n + 1][e] * inv,
                                                               od[n + 2][e] * inv, od[n + 3][e] * inv);
          } else {
#pragma unroll
            for (int n = 0; n < NTW; ++n) d0[n] = od[n][e] * inv;
          }
        }
      }
      if (cp == 0 && q == 0) a.part_lse[unit] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }
  };

  // Finished pieces whose partials wait in registers until the ring has drained.  A store
  // issued while block copies are in flight shares their counter: the waits for the next
  // blocks, which count only copies, would also wait for the store and leave the ring
  // with one block in flight for about two blocks.  Up to ND pieces wait this way (as
  // many as the registers allow at one workgroup per CU); a range with more stores the
  // later ones at once.  Pieces finish in order, so waiting piece k is piece k of the
  // plan, whose metadata stays in LDS.
  constexpr int ND = RT >= 4 ? 2 : 4;
  struct Done {
    f32x4 o[NTW];
    float m, l;
  };
  Done done[ND];
  int ndone = 0;
  auto finish_piece = [&]() {
    if (ndone < ND) {
#pragma unroll
      for (int k = 0; k < ND; ++k) {
        if (k == ndone) {
#pragma unroll
          for (int n = 0; n < NTW; ++n) done[k].o[n] = o[n];
          done[k].m = m_run;
          done[k].l = l_run;
        }
      }
      ++ndone;
    } else {
      store_partial(o, m_run, l_run, slot_c, row0_c, h_c, qo_c);
    }
  };

  auto begin_piece = [&](int k, int u) {
    h_c = __builtin_amdgcn_readfirstlane(sh.piece[k].h);
    row0_c = __builtin_amdgcn_readfirstlane(sh.piece[k].row0);
    qo_c = __builtin_amdgcn_readfirstlane(sh.piece[k].qo);
    const int kv = __builtin_amdgcn_readfirstlane(sh.piece[k].kv);
    slot_c = __builtin_amdgcn_readfirstlane(sh.piece[k].slot);
    const int nrows = qo_c * G;
    row_live = row < nrows;
    t_row = row_live ? row / G : 0;
    bound_row = row_live ? kv - qo_c + t_row + 1 : 0;
    first_bound = kv - qo_c + 1;
    all_tokens = qo_c >= 32 ? ~0 : (1 << qo_c) - 1;
    const char* qp = sh.qbuf + u * LdsT::QBYTES + row * D * 2 + q * (D / 4) * 2;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const uint4 w = row_live ? *reinterpret_cast<const uint4*>(qp + Gm::step_unit(q, s) * 16)
                               : make_uint4(0, 0, 0, 0);
      qb[s] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int n = 0; n < NTW; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  };

  // Prologue: blocks 0 .. kStages - 2 in flight.
  static_for<kStages - 1>([&](auto slot_c2) {
    if (decltype(slot_c2)::value < nblk) issue(slot_c2, decltype(slot_c2)::value);
  });

  auto step = [&](auto slot_cc, int j) {
    constexpr int u = decltype(slot_cc)::value;
    constexpr int un = (u + kStages - 1) % kStages;
    // This wave's LDS reads of block j - 1 are complete and its copies of block j (and
    // of the query rows issued with it) have landed; the barrier extends both facts to
    // every wave.  Later copies and output stores only make the count conservative.
    wait_lgkmcnt0();
    wait_blocks<Gm::LPT, kStages - 2>(min(nblk - 1 - j, kStages - 2));
    ring_barrier();
    if (j == c_next) {
      if (kc >= 0) finish_piece();
      ++kc;
      begin_piece(kc, u);
      c_next = __builtin_amdgcn_readfirstlane(sh.piece[kc + 1].start);
    }

    const char* kb = sh.ring + u * Gm::BLOCK;
    const char* vb = kb + Gm::HALF;
    bf16x8 kop[2][STEPS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < STEPS; ++s) kop[tt][s] = k_operand<D, KDT>(kb, tt, s, i, q);
    uint32_t vraw[8][4];
    v_runs<D, KDT, NTW>(vb, i, q, n0, vraw);

    const int pos0 = slot_pos[u];
    const int mask = slot_mask[u];
    const int kv = slot_kv[u];
    const int jn = j + kStages - 1;
    if (jn < nblk) issue(std::integral_constant<int, un>{}, jn);

    const bool inside = pos0 + kSub <= first_bound && (mask & all_tokens) == all_tokens;
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
    // The same lazy rescale as the ring kernel: the reference maximum moves only when a
    // score passes it by 2^8, and the cross-lane maximum runs only on a wave vote.
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
    if (pos0 + kSub > kv) v_zero_tail(q, pos0, kv, vraw);
#pragma unroll
    for (int n = 0; n < NTW; ++n) o[n] = mfma16(v_operand<KDT>(vraw, n), pb, o[n]);
  };

  for (int b0 = 0; b0 < nblk; b0 += kStages) {
    static_for<kStages>([&](auto slot_cc) {
      const int b = b0 + decltype(slot_cc)::value;
      if (b < nblk) step(slot_cc, b);
    });
  }

  // The waiting pieces go out from registers; the last piece through the ring, idle now,
  // as whole coalesced rows.
  wait_vmcnt<0>();
  __syncthreads();
#pragma unroll
  for (int k = 0; k < ND; ++k)
    if (k < ndone)
      store_partial(done[k].o, done[k].m, done[k].l,
                    __builtin_amdgcn_readfirstlane(sh.piece[k].slot),
                    __builtin_amdgcn_readfirstlane(sh.piece[k].row0),
                    __builtin_amdgcn_readfirstlane(sh.piece[k].h),
                    __builtin_amdgcn_readfirstlane(sh.piece[k].qo));
  constexpr int OPAD = D + 4;
  static_assert(LdsT::ROWS * OPAD * 4 <= kStages * Gm::BLOCK + kStages * LdsT::QBYTES,
                "output rows fit the ring and query buffers");
  float (*o_lds)[OPAD] = reinterpret_cast<float (*)[OPAD]>(sh.ring);
  float* l_lds = reinterpret_cast<float*>(sh.x);          // block indices are spent
  float* m_lds = l_lds + LdsT::ROWS;
  {
    float l = l_run + __shfl_xor(l_run, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (cp == 0 && q == 0) {
      l_lds[row] = l;
      m_lds[row] = m_run;
    }
#pragma unroll
    for (int n = 0; n < NTW; ++n)
#pragma unroll
      for (int e = 0; e < 4; ++e) o_lds[row][NT * (4 * q + e) + n0 + n] = o[n][e];
  }
  __syncthreads();
  const int nrows = qo_c * G;
  for (int item = tid; item < nrows * (D / 8); item += 256) {
    const int orow = item / (D / 8);
    const int c0 = (item - orow * (D / 8)) * 8;
    const int t = orow / G;
    const int64_t unit = (static_cast<int64_t>(slot_c) * rows_cap + row0_c + t) * a.num_q_heads +
                         h_c * G + (orow - t * G);
    const float L = l_lds[orow];
    if (L > 0.f) {
      const float inv = a.v_scale / L;
      float4* dst = reinterpret_cast<float4*>(a.part_o + unit * D + c0);
      dst[0] = make_float4(o_lds[orow][c0] * inv, o_lds[orow][c0 + 1] * inv,
                           o_lds[orow][c0 + 2] * inv, o_lds[orow][c0 + 3] * inv);
      dst[1] = make_float4(o_lds[orow][c0 + 4] * inv, o_lds[orow][c0 + 5] * inv,
                           o_lds[orow][c0 + 6] * inv, o_lds[orow][c0 + 7] * inv);
    }
    if (c0 == 0) a.part_lse[unit] = L > 0.f ? (m_lds[orow] + __log2f(L)) * kLn2 : -INFINITY;
  }
}

template <int RT, int D, int KDT, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
sdv_attn_flat_kernel(AttnArgs a, DenseSource ds, SparseSource ss) {
  static_assert(!is_sparse(MODE), "dense sources only");
  __shared__ FlatLds<RT, D, KDT> sh;
  const int tid = threadIdx.x;
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;
  const int S = a.num_splits;
  const int64_t rows_cap = static_cast<int64_t>(a.B) * a.max_qo_len;
  persistent_prefix<MODE>(sh.pl, a, ds, ss);
  const int L = __builtin_amdgcn_readfirstlane(sh.pl.seg_len);
  const int W = __builtin_amdgcn_readfirstlane(sh.pl.cum[a.B]) * Hkv;
  const int g = blockIdx.x;
  if (static_cast<int64_t>(g) * L >= W) return;
  const int begin = g * L;
  const int end = static_cast<int>(min<int64_t>(static_cast<int64_t>(begin) + L, W));
  int r = persistent_request(sh.pl, a.B, Hkv, begin);
  int pos = begin;
  bool planned_before = false;
  while (pos < end) {
    // ---- plan: the pieces of [pos, end), at most kFlatMaxPieces of them ----
    // (the ring has overwritten the request prefix since the last plan: rebuild it)
    if (planned_before) persistent_prefix<MODE>(sh.pl, a, ds, ss);
    planned_before = true;
    int npieces = 0, nblk = 0;
    while (pos < end && npieces < kFlatMaxPieces) {
      const int c0 = __builtin_amdgcn_readfirstlane(sh.pl.cum[r]);
      const int nb = __builtin_amdgcn_readfirstlane(sh.pl.cum[r + 1]) - c0;
      const int rstart = c0 * Hkv;
      if (nb == 0 || pos >= rstart + nb * Hkv) {
        ++r;
        continue;
      }
      const int h = (pos - rstart) / nb;
      const int pair0 = rstart + h * nb;
      const int stop = min(end, pair0 + nb);
      if (tid == 0) {
        FlatPiece& pc = sh.piece[npieces];
        pc.r = r;
        pc.h = h;
        pc.first = pos - pair0;
        pc.start = nblk;
        pc.slot = g - pair0 / L;
        pc.nb = nb;
      }
      nblk += stop - pos;
      ++npieces;
      pos = stop;
    }
    if (tid == 0) sh.piece[npieces].start = nblk;
    __syncthreads();
    for (int k = tid; k < npieces; k += 256) {
      const int rr = sh.piece[k].r;
      const int row0 = a.qo_indptr[rr];
      sh.piece[k].row0 = row0;
      sh.piece[k].qo = a.qo_indptr[rr + 1] - row0;
      sh.piece[k].kv = a.kv_len[rr];
    }
    // every block's page index (out of range: flagged, and the block is read masked out)
    for (int b = tid; b < nblk; b += 256) {
      int lo = 0, hi = npieces - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sh.piece[mid].start <= b) lo = mid;
        else hi = mid - 1;
      }
      const int rr = sh.piece[lo].r;
      const int pb = sh.piece[lo].first + (b - sh.piece[lo].start);
      int32_t xb;
      if constexpr (MODE == kSrcView) {
        int64_t xk, xv;
        const bool ok = view_pages(ds, rr, pb, xk, xv) && xv == xk + 4;
        if (!ok) set_err(a.dev_err, SDV_DEVERR_PAGE_RANGE);
        xb = ok ? static_cast<int32_t>(xk) : -1;
      } else {
        const int32_t phys = ss.block_table[static_cast<int64_t>(rr) * ss.bt_stride + (pb >> 2)];
        const bool ok = phys >= 0 && phys < ss.num_pages;
        if (!ok) set_err(a.dev_err, SDV_DEVERR_PAGE_RANGE);
        xb = ok ? phys : -1;
      }
      sh.x[b] = xb;
    }
    __syncthreads();
    flat_attend<RT, D, KDT, MODE>(sh, a, ds, ss, nblk);
    // pieces that end their pair: the pair's later split slots hold no keys (written after
    // the ring, so that no store is queued ahead of the first block copies)
    for (int k = 0; k < npieces; ++k) {
      const int nb = __builtin_amdgcn_readfirstlane(sh.piece[k].nb);
      const int n = __builtin_amdgcn_readfirstlane(sh.piece[k + 1].start) -
                    __builtin_amdgcn_readfirstlane(sh.piece[k].start);
      const int slot = __builtin_amdgcn_readfirstlane(sh.piece[k].slot);
      if (__builtin_amdgcn_readfirstlane(sh.piece[k].first) + n != nb) continue;
      const int h = __builtin_amdgcn_readfirstlane(sh.piece[k].h);
      const int row0 = __builtin_amdgcn_readfirstlane(sh.piece[k].row0);
      const int rows = __builtin_amdgcn_readfirstlane(sh.piece[k].qo) * G;
      for (int e = tid; e < (S - 1 - slot) * rows; e += 256) {
        const int kk = slot + 1 + e / rows;
        const int row = e % rows;
        const int t = row / G;
        a.part_lse[(kk * rows_cap + row0 + t) * a.num_q_heads + h * G + (row - t * G)] = -INFINITY;
      }
    }
    __syncthreads();   // LDS is planned again for the rest of the range
  }
}

template <int RT, int D, int KDT, int MODE>
hipError_t launch_t(const AttnArgs& a, const DenseSource& ds, const SparseSource& ss,
                    int64_t cap_blocks, hipStream_t s) {
  static const int per_cu = resident_per_cu(sdv_attn_flat_kernel<RT, D, KDT, MODE>);
  AttnArgs args = a;
  args.target_wgs = per_cu * device_cu_count();
  // enough workgroups for ranges of kMaxDenseBlocks when the balanced length is longer
  const int64_t need = (static_cast<int64_t>(a.B) * a.num_kv_heads * cap_blocks + kMaxDenseBlocks - 1) /
                       kMaxDenseBlocks;
  const int64_t wgs = std::max<int64_t>(args.target_wgs, need);
  hipLaunchKernelGGL((sdv_attn_flat_kernel<RT, D, KDT, MODE>), dim3(static_cast<uint32_t>(wgs)),
                     dim3(256), 0, s, args, ds, ss);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(const AttnArgs& a, const DenseSource& ds, const SparseSource& ss,
                    int64_t cap_blocks, hipStream_t s) {
  const int rows = a.max_qo_len * (a.num_q_heads / a.num_kv_heads);
  const int rt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
#define SDV_FLAT_CASE(RTV, DV, KDTV)                                                   \
  if (rt == RTV && a.head_dim == DV && a.kv_dt == KDTV)                                \
    return launch_t<RTV, DV, KDTV, MODE>(a, ds, ss, cap_blocks, s);
  SDV_FLAT_CASE(1, 128, SDV_BF16)
  SDV_FLAT_CASE(2, 128, SDV_BF16)
  SDV_FLAT_CASE(4, 128, SDV_BF16)
  SDV_FLAT_CASE(1, 64, SDV_BF16)
  SDV_FLAT_CASE(2, 64, SDV_BF16)
  SDV_FLAT_CASE(4, 64, SDV_BF16)
  SDV_FLAT_CASE(1, 128, SDV_FP8_E4M3)
  SDV_FLAT_CASE(2, 128, SDV_FP8_E4M3)
  SDV_FLAT_CASE(4, 128, SDV_FP8_E4M3)
  SDV_FLAT_CASE(1, 64, SDV_FP8_E4M3)
  SDV_FLAT_CASE(2, 64, SDV_FP8_E4M3)
  SDV_FLAT_CASE(4, 64, SDV_FP8_E4M3)
#undef SDV_FLAT_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_dense_flat(const AttnArgs& a, const DenseSource& src, hipStream_t s) {
  return dispatch<kSrcView>(a, src, SparseSource{}, src.max_sub_pages, s);
}

hipError_t launch_attn_paged_flat(const AttnArgs& a, const SparseSource& src, hipStream_t s) {
  return dispatch<kSrcPaged>(a, DenseSource{}, src, 4ll * src.max_pages, s);
}

}  // namespace sdv
