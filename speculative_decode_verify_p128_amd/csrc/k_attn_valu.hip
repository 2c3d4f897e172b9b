// Verify attention on the vector ALUs (any supported element type).
//
// Dense: token t of request r attends its request's positions j < bound(r,t) =
// kv_len - qo_len + t + 1, read through the P32 sub-page view ("[None][perf] Default
// Minimax-m3 to unified draft-target kv manager ...", Description and item 2).
// Sparse: token t, KV head h attends positions j < bound(r,t) whose page j / 128 it
// selected ("[TRTLLM-14093][feat] Eagle3 for M3 MSA path + CUDA graphs
// compatibility", MSA verify commit).  Unlike the pages' row-expanded kernel, every
// (request, KV head) reads the union of its tokens' pages once and applies each
// token's own page set as a per-row mask.
//
// One workgroup (256 threads) per (request, KV head, split).  Query rows are the G x
// qo (token, head) pairs, row = t * G + g, at most 64.  Keys and values pass through
// LDS in 16-token tiles as float; scores, online-softmax state and the output
// accumulators are float32; exponentials in base 2 with log2(e) folded into the
// query scale.
#include "device.h"
#include "internal.h"
#include "sparse_union.h"

namespace sdv {

constexpr int kMaxRows = 64;
constexpr int kTile = 16;

template <int D>
struct ValuSmem {
  float qs[kMaxRows][D];
  float ks[kTile][D + 1];
  float vs[kTile][D];
  float ps[kMaxRows][kTile];
  float row_m[kMaxRows];
  float row_l[kMaxRows];
  float row_a[kMaxRows];
  UnionLds u;
};

template <int D, bool SPARSE>
__global__ void __launch_bounds__(256) sdv_attn_valu_kernel(AttnArgs a, DenseSource ds,
                                                           SparseSource ss) {
  __shared__ ValuSmem<D> sm;
  constexpr int NE = kMaxRows * D / 256;   // accumulators per thread
  const int tid = threadIdx.x;
  // grid x = (request, KV head), y = split, the request rotated by the split, as in the
  // matrix-core kernels: no grid dimension bounds the batch size
  const int Hkv = a.num_kv_heads;
  const int split = blockIdx.y;
  const int h = blockIdx.x % Hkv;
  const int r = static_cast<int>((blockIdx.x / Hkv + split) % static_cast<uint32_t>(a.B));
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
  const int R = qo * G;
  const float qscale = a.softmax_scale * a.k_scale * kLog2e;

  // Query rows, scaled into the base-2 score domain.
  for (int i = tid; i < R * D; i += 256) {
    const int row = i / D;
    const int c = i - row * D;
    const int t = row / G;
    const int g = row - t * G;
    const int64_t src = (static_cast<int64_t>(row0 + t) * a.num_q_heads + h * G + g) * D + c;
    sm.qs[row][c] = load_elem(a.q, src, a.q_dt) * qscale;
  }
  if (tid < kMaxRows) {
    sm.row_m[tid] = -INFINITY;
    sm.row_l[tid] = 0.f;
  }

  // This split's work: a range of 32-token blocks.
  int blk_lo, blk_hi;     // dense: sub-pages; sparse: union entries (each 4 blocks)
  int n_union = 0;
  if constexpr (SPARSE) {
    n_union = build_union<false>(sm.u, ss, r, h, Hkv, row0, qo, kv, a.dev_err);
    const int chunk = (n_union + a.num_splits - 1) / a.num_splits;
    blk_lo = split * chunk;
    blk_hi = min(n_union, blk_lo + chunk);
  } else {
    const int chunk = (ds.max_sub_pages + a.num_splits - 1) / a.num_splits;
    const int nb = (kv + kSub - 1) / kSub;
    blk_lo = split * chunk;
    blk_hi = min(nb, blk_lo + chunk);
  }
  __syncthreads();

  float o[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) o[e] = 0.f;

  const int n_sub = SPARSE ? 4 : 1;    // 32-token blocks per work item
  for (int item = blk_lo; item < blk_hi; ++item) {
    int mask = ~0;
    const void* kb = nullptr;
    const void* vb = nullptr;
    int64_t kofs = 0, vofs = 0;     // element offset of token 0 of the 32-token block
    int pos_base;
    bool ok = true;
    if constexpr (SPARSE) {
      const int p = sm.u.upage[item];
      mask = sm.u.umask[item];
      const int phys = ss.block_table[static_cast<int64_t>(r) * ss.bt_stride + p];
      if (phys < 0 || phys >= ss.num_pages) ok = false;
      kb = ss.k;
      vb = ss.v;
      kofs = (static_cast<int64_t>(phys) * ss.page_stride + static_cast<int64_t>(h) * kPage * D);
      vofs = kofs;
      pos_base = p * kPage;
    } else {
      int64_t xk, xv;
      if (!view_pages(ds, r, item, xk, xv)) ok = false;
      kb = ds.root;
      vb = ds.root;
      kofs = (xk * Hkv + h) * kSub * D;
      vofs = (xv * Hkv + h) * kSub * D;
      pos_base = item * kSub;
    }
    if (!ok) {
      if (tid == 0) set_err(a.dev_err, SDV_DEVERR_PAGE_RANGE);
      continue;
    }
    for (int sb = 0; sb < n_sub; ++sb) {
      const int blk_pos = pos_base + sb * kSub;
      if (blk_pos >= kv) break;
      const int64_t kb_ofs = kofs + (SPARSE ? static_cast<int64_t>(sb) * kSub * D : 0);
      const int64_t vb_ofs = vofs + (SPARSE ? static_cast<int64_t>(sb) * kSub * D : 0);
      for (int half = 0; half < kSub / kTile; ++half) {
        const int tile_pos = blk_pos + half * kTile;
        if (tile_pos >= kv) break;
        for (int i = tid; i < kTile * D; i += 256) {
          const int jj = i / D;
          const int c = i - jj * D;
          const bool live = tile_pos + jj < kv;
          const int64_t off = static_cast<int64_t>(half * kTile + jj) * D + c;
          sm.ks[jj][c] = live ? load_elem(kb, kb_ofs + off, a.kv_dt) : 0.f;
          sm.vs[jj][c] = live ? load_elem(vb, vb_ofs + off, a.kv_dt) : 0.f;
        }
        __syncthreads();
        for (int i = tid; i < R * kTile; i += 256) {
          const int row = i / kTile;
          const int jj = i - row * kTile;
          const int t = row / G;
          const int pos = tile_pos + jj;
          const bool allowed = pos < kv - qo + t + 1 && ((mask >> t) & 1);
          float s = 0.f;
#pragma unroll 8
          for (int c = 0; c < D; ++c) s += sm.qs[row][c] * sm.ks[jj][c];
          sm.ps[row][jj] = allowed ? s : -INFINITY;
        }
        __syncthreads();
        if (tid < R) {
          const float m_old = sm.row_m[tid];
          float mx = m_old;
          for (int jj = 0; jj < kTile; ++jj) mx = fmaxf(mx, sm.ps[tid][jj]);
          float alpha = 1.f, lsum = 0.f;
          if (mx != -INFINITY) {
            alpha = exp2f(m_old - mx);
            for (int jj = 0; jj < kTile; ++jj) {
              const float pv = exp2f(sm.ps[tid][jj] - mx);
              sm.ps[tid][jj] = pv;
              lsum += pv;
            }
          } else {
            for (int jj = 0; jj < kTile; ++jj) sm.ps[tid][jj] = 0.f;
          }
          sm.row_a[tid] = alpha;
          sm.row_m[tid] = mx;
          sm.row_l[tid] = sm.row_l[tid] * alpha + lsum;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int idx = tid + 256 * e;
          const int row = idx / D;
          const int c = idx - row * D;
          if (row < R) {
            float acc = o[e] * sm.row_a[row];
            for (int jj = 0; jj < kTile; ++jj) acc += sm.ps[row][jj] * sm.vs[jj][c];
            o[e] = acc;
          }
        }
        __syncthreads();
      }
    }
  }

  // Write the (partial) result.
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int idx = tid + 256 * e;
    const int row = idx / D;
    const int c = idx - row * D;
    if (row >= R) continue;
    const int t = row / G;
    const int g = row - t * G;
    const int64_t qrow = row0 + t;
    const int hq = h * G + g;
    const float l = sm.row_l[row];
    const float val = l > 0.f ? o[e] * a.v_scale / l : 0.f;
    if (a.num_splits == 1) {
      store_out(a.out, (qrow * a.num_q_heads + hq) * D + c, val, a.out_dt);
    } else {
      const int64_t rows_cap = static_cast<int64_t>(a.B) * a.max_qo_len;
      const int64_t unit = (static_cast<int64_t>(split) * rows_cap + qrow) * a.num_q_heads + hq;
      a.part_o[unit * D + c] = val;
      if (c == 0) a.part_lse[unit] = l > 0.f ? (sm.row_m[row] + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

template <bool SPARSE>
static hipError_t launch_valu(const AttnArgs& a, const DenseSource& ds, const SparseSource& ss,
                              hipStream_t s) {
  dim3 grid(a.num_kv_heads * a.B, a.num_splits);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((sdv_attn_valu_kernel<128, SPARSE>), grid, dim3(256), 0, s, a, ds, ss);
  else
    hipLaunchKernelGGL((sdv_attn_valu_kernel<64, SPARSE>), grid, dim3(256), 0, s, a, ds, ss);
  return hipGetLastError();
}

hipError_t launch_attn_dense_valu(const AttnArgs& a, const DenseSource& src, hipStream_t s) {
  return launch_valu<false>(a, src, SparseSource{}, s);
}

hipError_t launch_attn_sparse_valu(const AttnArgs& a, const SparseSource& src, hipStream_t s) {
  return launch_valu<true>(a, DenseSource{}, src, s);
}

}  // namespace sdv
