// Verify attention on the CDNA4 matrix cores (bf16 queries; bf16 or fp8 K/V).
//
// What is computed: token t of request r, query head hq of KV head h attends the
// positions j < bound(r,t) = kv_len - qo_len + t + 1 ("[TRTLLM-14093][feat] Eagle3
// for M3 MSA path + CUDA graphs compatibility", MSA verify commit); dense keys come
// through the P32 sub-page view of the draft layer's P128 pages ("[None][perf]
// Default Minimax-m3 to unified draft-target kv manager ...", Description and item 2
// Grouped-HND), sparse keys only from the pages the token selected.  Float32
// accumulation; probabilities enter the value product as bf16.
//
// Layout of the work (gfx950, wave64, v_mfma_f32_16x16x32_bf16):
//   * A workgroup (4 waves) owns one (request, KV head, split).  Its query rows are the
//     G x qo (token, head) pairs (row = t * G + g), RT tiles of 16 rows.  Every wave
//     keeps all RT row tiles and takes every fourth 32-token block of the split, so a
//     K/V byte is loaded by exactly one wave, straight from HBM into registers.
//   * Scores are computed transposed, S^T = K Q^T: K is the A operand (lane l holds
//     token l % 16 and 8 consecutive channels of a 32-channel step), Q^T the B operand
//     (kept in registers for the whole kernel).  The result leaves lane l holding
//     query row l % 16 for tokens 4(l/16) .. +3 of each 16-token tile — exactly the B
//     operand layout the value product needs, so O^T = V^T P^T follows with no data
//     exchange.  O^T keeps each query row in one lane, so the online-softmax rescale
//     is a per-lane multiply.
//   * Channels inside a 32-channel step are permuted (lane group q handles channels
//     q * d/4 .. q * d/4 + d/4 - 1 across the steps) so each lane's K bytes are one
//     contiguous run; Q uses the same permutation, leaving the dot products unchanged.
//     V is read as 16-byte (bf16) runs of d/16 channels per token and transposed in
//     registers into the A operand with byte permutes.
//   * The next block's K/V loads are issued before the current block is computed.
//   * At the end the four waves merge (max, sum, output) through LDS in a fixed
//     order, and the workgroup writes the output, or a normalised partial and its
//     log-sum-exp for the split-KV combine.
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

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int W>
__device__ __forceinline__ void load_words(const char* p, uint32_t* dst) {
  if constexpr (W == 4) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
  } else if constexpr (W == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    dst[0] = x.x; dst[1] = x.y;
  } else {
    dst[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

// What one lane loads of a 32-token block.
template <int D, int KDT>
struct Raw {
  static constexpr int STEPS = D / 32;            // 32-channel MFMA steps
  static constexpr int NT = D / 16;               // 16-channel output tiles
  static constexpr int EB = elem_bytes<KDT>();
  static constexpr int KW = 8 * EB / 4;           // words per (tile, step): 8 channels
  static constexpr int VW = NT * EB / 4;          // words per token: NT channels
  uint32_t k[2][STEPS][KW];
  uint32_t v[8][VW];
};

// Token of the 32-token block that element e (0..7) of lane group q stands for in the
// value product: the score tile of tokens 0-15 gives e < 4, the one of 16-31 e >= 4.
__device__ __forceinline__ int ptok(int q, int e) { return e < 4 ? 4 * q + e : 12 + 4 * q + e; }

template <int D, int KDT>
__device__ __forceinline__ void load_block(Raw<D, KDT>& raw, const char* kp, const char* vp,
                                           int i, int q) {
  using R = Raw<D, KDT>;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int s = 0; s < R::STEPS; ++s)
      load_words<R::KW>(kp + (tt * 16 + i) * D * R::EB + (q * (D / 4) + s * 8) * R::EB,
                        raw.k[tt][s]);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    load_words<R::VW>(vp + ptok(q, e) * D * R::EB + R::NT * i * R::EB, raw.v[e]);
}

template <int D, int KDT>
__device__ __forceinline__ bf16x8 k_operand(const Raw<D, KDT>& raw, int tt, int s) {
  if constexpr (KDT == SDV_BF16) {
    uint4 w = make_uint4(raw.k[tt][s][0], raw.k[tt][s][1], raw.k[tt][s][2], raw.k[tt][s][3]);
    return __builtin_bit_cast(bf16x8, w);
  } else {
    float f[8];
    fp8x2_to_f32<false>(raw.k[tt][s][0], f[0], f[1]);
    fp8x2_to_f32<true>(raw.k[tt][s][0], f[2], f[3]);
    fp8x2_to_f32<false>(raw.k[tt][s][1], f[4], f[5]);
    fp8x2_to_f32<true>(raw.k[tt][s][1], f[6], f[7]);
    uint4 w = make_uint4(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]),
                         pack2_bf16(f[4], f[5]), pack2_bf16(f[6], f[7]));
    return __builtin_bit_cast(bf16x8, w);
  }
}

// A operand of O^T += V^T P^T for output tile n: element e = V[ptok(q, e)][NT*i + n].
template <int D, int KDT>
__device__ __forceinline__ bf16x8 v_operand(const Raw<D, KDT>& raw, int n) {
  using R = Raw<D, KDT>;
  uint32_t w[4];
  if constexpr (KDT == SDV_BF16) {
    const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      w[m] = __builtin_amdgcn_perm(raw.v[2 * m + 1][n >> 1], raw.v[2 * m][n >> 1], sel);
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float a0, a1, b0, b1;
      const uint32_t wa = raw.v[2 * m][n >> 2];
      const uint32_t wb = raw.v[2 * m + 1][n >> 2];
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
  (void)sizeof(R);
  return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// One 32-token block: scores, online-softmax update and value product for all RT row
// tiles of this lane.  cur_pos0 is the block's first position in the request,
// cur_mask the verify tokens that selected it (all for dense).
template <int RT, int D, int KDT>
__device__ __forceinline__ void compute_block(Raw<D, KDT>& cur, int cur_pos0, int cur_mask,
                                              int kv, int q, const int (&t_row)[RT],
                                              const int (&bound_row)[RT],
                                              const bf16x8 (&qb)[RT][D / 32], float qk_scale,
                                              f32x4 (&o)[RT][D / 16], float (&m)[RT],
                                              float (&l)[RT]) {
  using R = Raw<D, KDT>;
  constexpr int STEPS = R::STEPS;
  constexpr int NT = R::NT;
  // Values of positions beyond kv_len are zeroed: stale storage must not reach P * V.
  if (cur_pos0 + kSub > kv) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (cur_pos0 + ptok(q, e) >= kv)
#pragma unroll
        for (int w = 0; w < R::VW; ++w) cur.v[e][w] = 0u;
  }
  bf16x8 pb[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    f32x4 sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < STEPS; ++s)
        sacc[tt] = mfma16(k_operand<D, KDT>(cur, tt, s), qb[rt][s], sacc[tt]);
    }
    const int bnd = ((cur_mask >> t_row[rt]) & 1) ? bound_row[rt] : 0;
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = cur_pos0 + tt * 16 + 4 * q + e;
        const float sv = pos < bnd ? sacc[tt][e] * qk_scale : -INFINITY;
        sacc[tt][e] = sv;
        mx = fmaxf(mx, sv);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m[rt], mx);
    float p[8];
    float alpha = 1.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = 0.f;
    } else {
      alpha = __builtin_amdgcn_exp2f(m[rt] - m_new);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = __builtin_amdgcn_exp2f(sacc[0][e] - m_new);
        p[e + 4] = __builtin_amdgcn_exp2f(sacc[1][e] - m_new);
      }
    }
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ls += p[e];
    l[rt] = l[rt] * alpha + ls;
    m[rt] = m_new;
    pb[rt] = __builtin_bit_cast(bf16x8, make_uint4(pack2_bf16(p[0], p[1]), pack2_bf16(p[2], p[3]),
                                                   pack2_bf16(p[4], p[5]), pack2_bf16(p[6], p[7])));
    if (alpha != 1.f) {
#pragma unroll
      for (int n = 0; n < NT; ++n) o[rt][n] *= alpha;
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const bf16x8 va = v_operand<D, KDT>(cur, n);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) o[rt][n] = mfma16(va, pb[rt], o[rt][n]);
  }
}

struct NoUnion {};

template <int RT, int D, int KDT, bool SPARSE>
__global__ void __launch_bounds__(256) sdv_attn_mfma_kernel(AttnArgs a, DenseSource ds,
                                                           SparseSource ss) {
  using R = Raw<D, KDT>;
  constexpr int STEPS = R::STEPS;
  constexpr int NT = R::NT;
  constexpr int ROWS = RT * 16;
  constexpr int OPAD = D + 4;
  constexpr int EB = R::EB;
  __shared__ float o_lds[ROWS][OPAD];
  __shared__ float m_lds[4][ROWS];
  __shared__ float l_lds[4][ROWS];
  __shared__ float L_lds[ROWS];
  __shared__ float M_lds[ROWS];
  __shared__ typename std::conditional<SPARSE, UnionLds, NoUnion>::type ul;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int i = lane & 15;
  const int q = lane >> 4;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int r = blockIdx.z;
  const int Hkv = a.num_kv_heads;
  const int G = a.num_q_heads / Hkv;

  const int64_t kv_cap = SPARSE ? static_cast<int64_t>(ss.max_pages) * kPage
                                : static_cast<int64_t>(ds.max_sub_pages) * kSub;
  const int row0 = a.qo_indptr[r];
  const int qo = a.qo_indptr[r + 1] - row0;
  const int kv = a.kv_len[r];
  const bool bad_len = qo < 1 || qo > a.max_qo_len || kv < qo || row0 < 0 ||
                       static_cast<int64_t>(row0) + qo > static_cast<int64_t>(a.B) * a.max_qo_len;
  const bool bad_cap = !bad_len && kv > kv_cap;
  if (bad_len || bad_cap) {
    if (tid == 0 && split == 0 && h == 0)
      set_err(a.dev_err, bad_len ? SDV_DEVERR_QO_LEN : SDV_DEVERR_KV_CAPACITY);
    return;
  }
  const int nrows = qo * G;

  // Per row tile: this lane's query row, its token and its ladder bound.
  int t_row[RT], bound_row[RT];
  bf16x8 qb[RT][STEPS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + i;
    const bool live = row < nrows;
    const int t = live ? row / G : 0;
    const int g = live ? row - t * G : 0;
    t_row[rt] = t;
    bound_row[rt] = live ? kv - qo + t + 1 : 0;
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(row0 + t) * a.num_q_heads + h * G + g) * D +
                      q * (D / 4)) * 2;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      uint4 w = live ? *reinterpret_cast<const uint4*>(qp + s * 16) : make_uint4(0, 0, 0, 0);
      qb[rt][s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const float qk_scale = a.softmax_scale * a.k_scale * kLog2e;

  // This split's blocks; wave w takes blocks w, w + 4, ...
  int nblk, base;
  if constexpr (SPARSE) {
    const int n_union = build_union<false>(ul, ss, r, h, Hkv, row0, qo, kv, a.dev_err);
    const int chunk = (n_union + a.num_splits - 1) / a.num_splits;
    base = split * chunk;
    nblk = 4 * max(0, min(n_union, base + chunk) - base);
  } else {
    const int chunk = (ds.max_sub_pages + a.num_splits - 1) / a.num_splits;
    const int nb = (kv + kSub - 1) / kSub;
    base = split * chunk;
    nblk = max(0, min(nb, base + chunk) - base);
  }

  // Resolves block j of the split: K/V byte pointers, first position, token mask.
  auto locate = [&](int j, const char*& kp, const char*& vp, int& pos0, int& mask) -> bool {
    if constexpr (SPARSE) {
      const int e = base + (j >> 2);
      const int quarter = j & 3;
      const int p = ul.upage[e];
      mask = ul.umask[e];
      pos0 = p * kPage + quarter * kSub;
      if (pos0 >= kv) return false;
      const int phys = ss.block_table[static_cast<int64_t>(r) * ss.bt_stride + p];
      if (phys < 0 || phys >= ss.num_pages) {
        set_err(a.dev_err, SDV_DEVERR_PAGE_RANGE);
        return false;
      }
      const int64_t off = (static_cast<int64_t>(phys) * ss.page_stride +
                           (static_cast<int64_t>(h) * kPage + quarter * kSub) * D) * EB;
      kp = reinterpret_cast<const char*>(ss.k) + off;
      vp = reinterpret_cast<const char*>(ss.v) + off;
      return true;
    } else {
      const int x = base + j;
      int64_t xk, xv;
      mask = ~0;
      pos0 = x * kSub;
      if (!view_pages(ds, r, x, xk, xv)) {
        set_err(a.dev_err, SDV_DEVERR_PAGE_RANGE);
        return false;
      }
      kp = reinterpret_cast<const char*>(ds.root) + (xk * Hkv + h) * kSub * D * EB;
      vp = reinterpret_cast<const char*>(ds.root) + (xv * Hkv + h) * kSub * D * EB;
      return true;
    }
  };

  f32x4 o[RT][NT];
  float m[RT], l[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.f;
#pragma unroll
    for (int n = 0; n < NT; ++n) o[rt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Blocks of this wave (w, w + 4, ...); the next block's loads are issued before the
  // current block is computed.
  int j = wave;
  const char *kp = nullptr, *vp = nullptr;
  int pos0 = 0, mask = 0;
  bool have = false;
  while (j < nblk && !(have = locate(j, kp, vp, pos0, mask))) j += 4;
  Raw<D, KDT> cur;
  if (have) load_block<D, KDT>(cur, kp, vp, i, q);
  while (have) {
    const int cur_pos0 = pos0;
    const int cur_mask = mask;
    bool have_n = false;
    j += 4;
    while (j < nblk && !(have_n = locate(j, kp, vp, pos0, mask))) j += 4;
    Raw<D, KDT> nxt;
    if (have_n) load_block<D, KDT>(nxt, kp, vp, i, q);
    compute_block<RT, D, KDT>(cur, cur_pos0, cur_mask, kv, q, t_row, bound_row, qb, qk_scale, o,
                              m, l);
    have = have_n;
    if (have) cur = nxt;
  }

  // ---- merge the four waves (fixed order) ----
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l[rt] += __shfl_xor(l[rt], 16, kWave);
    l[rt] += __shfl_xor(l[rt], 32, kWave);
    if (q == 0) {
      m_lds[wave][rt * 16 + i] = m[rt];
      l_lds[wave][rt * 16 + i] = l[rt];
    }
  }
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + i;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, m_lds[w][row]);
    float sc = 0.f;
    if (M != -INFINITY && m[rt] != -INFINITY) sc = __builtin_amdgcn_exp2f(m[rt] - M);
    if (wave == 0 && q == 0) {
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (m_lds[w][row] != -INFINITY) L += l_lds[w][row] * __builtin_amdgcn_exp2f(m_lds[w][row] - M);
      L_lds[row] = L;
      M_lds[row] = M;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) o[rt][n] *= sc;
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float* dst = &o_lds[rt * 16 + i][0];
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ch = NT * (4 * q + e) + n;
            dst[ch] = (w == 0) ? o[rt][n][e] : dst[ch] + o[rt][n][e];
          }
      }
    }
    __syncthreads();
  }

  // ---- write out: 8 channels per thread item ----
  const int64_t rows_cap = static_cast<int64_t>(a.B) * a.max_qo_len;
  for (int item = tid; item < nrows * (D / 8); item += 256) {
    const int row = item / (D / 8);
    const int c0 = (item - row * (D / 8)) * 8;
    const int t = row / G;
    const int g = row - t * G;
    const int hq = h * G + g;
    const int64_t qrow = row0 + t;
    const float L = L_lds[row];
    const float inv = L > 0.f ? a.v_scale / L : 0.f;
    float v8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v8[e] = o_lds[row][c0 + e] * inv;
    if (a.num_splits == 1) {
      const int64_t idx = (qrow * a.num_q_heads + hq) * D + c0;
      if (a.out_dt == SDV_BF16) {
        uint4 w = make_uint4(pack2_bf16(v8[0], v8[1]), pack2_bf16(v8[2], v8[3]),
                             pack2_bf16(v8[4], v8[5]), pack2_bf16(v8[6], v8[7]));
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + idx) = w;
      } else {
        float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + idx);
        dst[0] = make_float4(v8[0], v8[1], v8[2], v8[3]);
        dst[1] = make_float4(v8[4], v8[5], v8[6], v8[7]);
      }
    } else {
      const int64_t unit = (static_cast<int64_t>(split) * rows_cap + qrow) * a.num_q_heads + hq;
      float4* dst = reinterpret_cast<float4*>(a.part_o + unit * D + c0);
      dst[0] = make_float4(v8[0], v8[1], v8[2], v8[3]);
      dst[1] = make_float4(v8[4], v8[5], v8[6], v8[7]);
      if (c0 == 0)
        a.part_lse[unit] = L > 0.f ? (M_lds[row] + __log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

template <int RT, int D, int KDT, bool SPARSE>
hipError_t launch_t(const AttnArgs& a, const DenseSource& ds, const SparseSource& ss,
                    hipStream_t s) {
  dim3 grid(a.num_splits, a.num_kv_heads, a.B);
  hipLaunchKernelGGL((sdv_attn_mfma_kernel<RT, D, KDT, SPARSE>), grid, dim3(256), 0, s, a, ds, ss);
  return hipGetLastError();
}

template <bool SPARSE>
hipError_t dispatch(const AttnArgs& a, const DenseSource& ds, const SparseSource& ss,
                    hipStream_t s) {
  const int rows = a.max_qo_len * (a.num_q_heads / a.num_kv_heads);
  const int rt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
#define SDV_MFMA_CASE(RTV, DV, KDTV)                                                   \
  if (rt == RTV && a.head_dim == DV && a.kv_dt == KDTV)                                \
    return launch_t<RTV, DV, KDTV, SPARSE>(a, ds, ss, s);
  SDV_MFMA_CASE(1, 128, SDV_BF16)
  SDV_MFMA_CASE(2, 128, SDV_BF16)
  SDV_MFMA_CASE(4, 128, SDV_BF16)
  SDV_MFMA_CASE(1, 64, SDV_BF16)
  SDV_MFMA_CASE(2, 64, SDV_BF16)
  SDV_MFMA_CASE(4, 64, SDV_BF16)
  SDV_MFMA_CASE(1, 128, SDV_FP8_E4M3)
  SDV_MFMA_CASE(2, 128, SDV_FP8_E4M3)
  SDV_MFMA_CASE(4, 128, SDV_FP8_E4M3)
  SDV_MFMA_CASE(1, 64, SDV_FP8_E4M3)
  SDV_MFMA_CASE(2, 64, SDV_FP8_E4M3)
  SDV_MFMA_CASE(4, 64, SDV_FP8_E4M3)
#undef SDV_MFMA_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool mfma_supported(const AttnArgs& a) {
  const bool aligned = (reinterpret_cast<uintptr_t>(a.q) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(a.out) % 16 == 0);
  return a.q_dt == SDV_BF16 && (a.kv_dt == SDV_BF16 || a.kv_dt == SDV_FP8_E4M3) &&
         (a.head_dim == 64 || a.head_dim == 128) &&
         a.max_qo_len * (a.num_q_heads / a.num_kv_heads) <= 64 && aligned;
}

hipError_t launch_attn_dense_mfma(const AttnArgs& a, const DenseSource& src, hipStream_t s) {
  return dispatch<false>(a, src, SparseSource{}, s);
}

hipError_t launch_attn_sparse_mfma(const AttnArgs& a, const SparseSource& src, hipStream_t s) {
  return dispatch<true>(a, DenseSource{}, src, s);
}

}  // namespace sdv
