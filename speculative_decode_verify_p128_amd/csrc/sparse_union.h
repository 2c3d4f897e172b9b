// Union of the pages a request's verify tokens selected for one KV head, built in LDS
// by a 256-thread workgroup.
//
// Each (request, KV head) reads every page that any of its tokens selected once; a
// per-page bit mask records which tokens selected it, and each token's rows attend
// only the pages whose bit is set (plus its ladder bound).  The list is sorted by
// request-local page number, which makes split-KV partitioning deterministic.
#pragma once

#include "device.h"
#include "internal.h"

namespace sdv {

constexpr int kMaxUnion = 512;   // max_qo_len * top_k
constexpr int kMaxWords = 512;   // max_pages <= 16384

struct UnionLds {
  uint32_t bitmap[kMaxWords];
  int32_t word_prefix[kMaxWords];
  int32_t upage[kMaxUnion];     // request-local page number
  int32_t uphys[kMaxUnion];     // physical page (0 when out of range, then umask = 0)
  int32_t umask[kMaxUnion];     // bit t: verify token t selected the page
  int32_t sel[kMaxUnion];       // in-kernel selection: [t][k] page, -1 padded
  int32_t scan[256];
};

static_assert(4 * kWave <= kMaxUnion, "the selection's staging fits the union's page arrays");

// One wave selects the k_eff = min(top_k, n) <= 64 best of srow[0 .. n-1] by the bit
// search and writes them to lout, in rank order when gout is non-null (and to gout too);
// returns k_eff.  Without gout the selection only feeds the page union, which does not
// depend on the order, so the pages go to lout unsorted: each selected key to its slot
// among the keys >= T (no bitonic network, no staging round trip through LDS).
template <int ITEMS>
__device__ __forceinline__ int wave_bits_select(const float* srow, int n, int top_k, int lane,
                                                uint32_t* st_hi, uint32_t* st_lo, int32_t* lout,
                                                int32_t* gout) {
  uint64_t key[ITEMS];
  wave_topk_keys(srow, n, lane, key);
  const int k_eff = top_k < n ? top_k : n;
  const uint64_t T = wave_kth_key(key, n, k_eff);
  if (!gout) {
    uint32_t pos = wave_selection_offset(key, T, lane);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      if (key[i] >= T) lout[pos++] = topk_key_page(key[i]);
    return k_eff;
  }
  const uint64_t v = wave_ranked_selection(key, T, lane, k_eff, st_hi, st_lo);
  if (lane < k_eff) {
    const int page = topk_key_page(v);
    lout[lane] = page;
    if (gout) gout[lane] = page;
  }
  return k_eff;
}

// Whether a token with n valid pages selects by the bit search when its ranked selection
// is written out too (WIDE kernels only): its cost does not grow with top_k, while the
// repeated maximum costs about top_k x (items + 8) dependent instructions; with top_k <=
// 64 the mark is passed from 11 key slots a lane (over 640 pages) on.  Measured on 8
// requests of 131072 fp8 tokens (1024 pages), top-64: the fused selection and attention
// 85.6 -> 68.2 us at 16 splits (66.6 -> 61.5 us once the search stops early and feeds the
// union unsorted).  A selection that only feeds the union takes the bit search whenever
// top_k <= 64 and n > top_k, since no sort follows it then (64 x U[4096, 32768] tokens,
// top-16: 146.0 -> 145.0 us for the fused call; a ragged batch 239.2 -> 238.4 us).
__host__ __device__ constexpr bool select_by_bits(int n, int top_k) {
  return n > 4 * kWave && top_k <= kWave && top_k * ((n + kWave - 1) / kWave + 8) > 1200;
}

// Launches whose tables can hold such a token take the kernel variant that carries the
// bit search (the others keep the smaller code of the repeated maximum alone).
inline bool select_wide(const SparseSource& ss) { return select_by_bits(ss.max_pages, ss.top_k); }

// The ladder top-k of every verify token of (r, h) from ss.scores, one wave per token,
// into u.sel (and ss.topk_out / ss.cnt_out when non-null and write_out): the same
// selection as the top-k kernel.  All 256 threads call; ends with a barrier.
template <bool WIDE>
__device__ inline void select_topk(UnionLds& u, const SparseSource& ss, int h, int Hkv, int row0,
                                   int qo, int kv, bool write_out) {
  static_assert(kFusedTopkMaxPages == 16 * kWave, "item counts below");
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  for (int t = wave; t < qo; t += 256 / kWave) {
    const int n = (kv - qo + t + 1 + kPage - 1) / kPage;
    const int64_t unit = static_cast<int64_t>(row0 + t) * Hkv + h;
    const float* srow = ss.scores + unit * ss.max_pages;
    int32_t* gout = write_out && ss.topk_out ? ss.topk_out + unit * ss.top_k : nullptr;
    int32_t* lout = u.sel + t * ss.top_k;
    auto emit = [&](int k, int page) {
      if (lane == 0) {
        lout[k] = page;
        if (gout) gout[k] = page;
      }
    };
    // register slots per lane sized to this token's pages (each round rescans them)
    const int items = (n + kWave - 1) / kWave;
    int k_eff;
    // the keys are gathered through the union's page arrays, filled only after the
    // selection
    uint32_t* st_hi = reinterpret_cast<uint32_t*>(u.upage) + wave * kWave;
    uint32_t* st_lo = reinterpret_cast<uint32_t*>(u.uphys) + wave * kWave;
    if (WIDE && select_by_bits(n, ss.top_k)) {
      k_eff = wave_bits_select<16>(srow, n, ss.top_k, lane, st_hi, st_lo, lout, gout);
    } else if (!gout && ss.top_k <= kWave && n > ss.top_k) {
      // feeding the union only (no ranked output): the bit search, which stops after
      // about 14 rounds on real-valued scores, against top_k rounds of the maximum
      if (items <= 1) k_eff = wave_bits_select<1>(srow, n, ss.top_k, lane, st_hi, st_lo, lout, gout);
      else if (items <= 2) k_eff = wave_bits_select<2>(srow, n, ss.top_k, lane, st_hi, st_lo, lout, gout);
      else if (items <= 4) k_eff = wave_bits_select<4>(srow, n, ss.top_k, lane, st_hi, st_lo, lout, gout);
      else if (items <= 8) k_eff = wave_bits_select<8>(srow, n, ss.top_k, lane, st_hi, st_lo, lout, gout);
      else k_eff = wave_bits_select<16>(srow, n, ss.top_k, lane, st_hi, st_lo, lout, gout);
    } else if (items <= 1) k_eff = wave_ladder_topk<1>(srow, n, ss.top_k, lane, emit);
    else if (items <= 2) k_eff = wave_ladder_topk<2>(srow, n, ss.top_k, lane, emit);
    else if (items <= 4) k_eff = wave_ladder_topk<4>(srow, n, ss.top_k, lane, emit);
    else if (items <= 8) k_eff = wave_ladder_topk<8>(srow, n, ss.top_k, lane, emit);
    else k_eff = wave_ladder_topk<16>(srow, n, ss.top_k, lane, emit);
    for (int k = k_eff + lane; k < ss.top_k; k += kWave) {
      lout[k] = -1;
      if (gout) gout[k] = -1;
    }
    if (write_out && ss.cnt_out && lane == 0) ss.cnt_out[unit] = k_eff;
  }
  __syncthreads();
}

// All 256 threads must call.  Returns the number of distinct selected pages; flags
// (and ignores) indices at or beyond a token's valid-page count.  The pages come from
// ss.topk_idx, or (SELECT) from the in-kernel selection of ss.scores, written out to
// ss.topk_out / ss.cnt_out when write_out (WIDE: by the bit search where it pays).
template <bool SELECT, bool WIDE = false>
__device__ inline int build_union(UnionLds& u, const SparseSource& ss, int r, int h, int Hkv,
                                  int row0, int qo, int kv, int32_t* dev_err,
                                  bool write_out = false) {
  const int tid = threadIdx.x;
  const int words = (ss.max_pages + 31) / 32;
  if constexpr (SELECT) select_topk<WIDE>(u, ss, h, Hkv, row0, qo, kv, write_out);
  auto selected = [&](int t, int k) {
    if constexpr (SELECT) return u.sel[t * ss.top_k + k];
    else return ss.topk_idx[(static_cast<int64_t>(row0 + t) * Hkv + h) * ss.top_k + k];
  };
  for (int w = tid; w < words; w += 256) u.bitmap[w] = 0u;
  // This thread's (token, rank) elements, e = tid and tid + 256 (qo * top_k <= 512): the
  // page of each, or -1 when it selects none or is out of the token's range (flagged).
  static_assert(kMaxUnion <= 2 * 256, "two selection elements a thread");
  const int n_el = qo * ss.top_k;
  int el_page[2], el_tok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 256 * i;
    el_page[i] = -1;
    el_tok[i] = 0;
    if (e < n_el) {
      const int t = e / ss.top_k;
      const int p = selected(t, e - t * ss.top_k);
      const int nvalid = (kv - qo + t + 1 + kPage - 1) / kPage;
      if (p >= nvalid) set_err(dev_err, SDV_DEVERR_TOPK_INDEX);
      el_page[i] = p >= 0 && p < nvalid ? p : -1;
      el_tok[i] = t;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (el_page[i] >= 0) atomicOr(&u.bitmap[el_page[i] >> 5], 1u << (el_page[i] & 31));
  __syncthreads();
  // exclusive prefix of per-word popcounts; each thread owns two consecutive words: a
  // prefix inside each wave by lane shuffles, then the waves' totals
  const int w0 = 2 * tid;
  const int c0 = (w0 < words) ? __popc(u.bitmap[w0]) : 0;
  const int c1 = (w0 + 1 < words) ? __popc(u.bitmap[w0 + 1]) : 0;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  int inc = c0 + c1;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += v;
  }
  if (lane == kWave - 1) u.scan[wv] = inc;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int k = 0; k < 256 / kWave; ++k) {
    const int tw = u.scan[k];
    base += k < wv ? tw : 0;
    total += tw;
  }
  const int excl = base + inc - (c0 + c1);
  if (w0 < words) u.word_prefix[w0] = excl;
  if (w0 + 1 < words) u.word_prefix[w0 + 1] = excl + c0;
  __syncthreads();
  for (int w = tid; w < words; w += 256) {
    uint32_t bits = u.bitmap[w];
    int idx = u.word_prefix[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      u.upage[idx] = w * 32 + b;
      u.umask[idx] = 0;
      ++idx;
      bits &= bits - 1;
    }
  }
  __syncthreads();
  // every union entry's block-table entry at once (one memory round trip, not one per
  // page a thread's words hold)
  for (int e = tid; e < total; e += 256) {
    int phys = ss.block_table[static_cast<int64_t>(r) * ss.bt_stride + u.upage[e]];
    if (phys < 0 || phys >= ss.num_pages) {
      set_err(dev_err, SDV_DEVERR_PAGE_RANGE);
      phys = -1;
    }
    u.uphys[e] = phys;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = el_page[i];
    if (p < 0) continue;
    const int w = p >> 5;
    const int idx = u.word_prefix[w] + __popc(u.bitmap[w] & ((1u << (p & 31)) - 1u));
    if (u.uphys[idx] >= 0) atomicOr(&u.umask[idx], 1 << el_tok[i]);
  }
  __syncthreads();
  // Pages outside the pool keep an empty token mask and read page 0 (in bounds); the
  // request is flagged.
  for (int e = tid; e < total; e += 256)
    if (u.uphys[e] < 0) u.uphys[e] = 0;
  __syncthreads();
  return total;
}

}  // namespace sdv
