// Proxy page scores of the block-sparse target layer.
//
// "[TRTLLM-14093][feat] Eagle3 for M3 MSA path + CUDA graphs compatibility", MSA
// multi-token verify commit: the proxy ("OnlyScore") pass runs natively multi-token
// under the inclusive causal bound with offset kv_len - qo_len, so token t sees
// kv_len - qo_len + t + 1 positions.  The pages give no formula; this library scores
//   score(t, h, p) = max_{hq in group h} q[t, hq] . ksum(t, h, p),
//   ksum(t, h, p)  = sum of K[j, h, :] over positions j of page p with j < bound_t,
// in a fixed float32 order so that the ranking is reproducible bit for bit:
//   1. ksum accumulated one position at a time, ascending, from 0;
//   2. products q[c] * ksum[c] rounded separately (no fused multiply-add);
//   3. recursive halving over channels: u[c] += u[c + n/2] for n = d, d/2, ..., 2;
//   4. maximum over the G query heads; -0 becomes +0.
//
// Design (HBM-bound; K of every valid page is read exactly once for all tokens):
//   one workgroup = four waves per (request, KV head, run of 4 x 64/LPR pages); a group of LPR
//   lanes owns one page, each lane a contiguous slice of every key row (16 bytes: 8 bf16
//   or 4 f32 channels; 8 bytes: 8 fp8 channels), so each wave load instruction reads
//   64/LPR full page rows.  fp8 takes 8-byte slices so that a wave holds four pages rather
//   than eight: on 8 x 131072 fp8 tokens (32 pairs of 1024 pages) the 16-byte form fills
//   the GPU with exactly one generation of waves and nothing evens out their finishing
//   times (104.9 against 98.3 us, same scores bit for bit); 4-byte slices, two pages a
//   wave and four generations, measured slower again (101 against 98.5 us). (bf16 in
//   8-byte slices, two pages a wave, measured slower: 208 against 205 us on 64 x
//   U[4096, 32768] tokens, 230 against 180 us on a ragged batch.)  Four waves a workgroup
//   share one staging of the queries and make a quarter of the workgroups: against one
//   wave 198 -> 195 us on 64 x U[4096, 32768] bf16 tokens, 97.7 -> 94.8 us on 8 x 131072
//   fp8 tokens, 159.6 -> 156.9 us on a ragged batch (two waves: 198, 97, 157; eight: 204,
//   94, 162: past a short request's last page the waves of a large workgroup idle, and
//   its LDS stays held until they all end).  Each lane keeps 256 bytes of rows in flight (16 rows
//   of 16-byte slices, 32 of 8-byte: fp8 with 16 rows measured 2.8% slower); the loads are
//   non-temporal (the keys are read once, so they should not displace what the caches
//   hold), which measured about 20% faster than ordinary loads on this streaming pattern.
//   A lane keeps its channels' running sums in registers and scores a token as soon as the
//   running sum reaches that token's bound; the tokens' bounds differ by one position, so
//   every token shares one pass. The halving tree first pairs channels c and c + d/2,
//   which live in different lanes of the group (DPP row shifts inside 16-lane rows), and
//   ends inside the lane. Granularity matters more than per-wave start-up: four pages per
//   wave measured faster than eight or sixteen streamed one after another by the same
//   lanes, and keeping the next 8 rows in flight while 8 are added (up to 24 per lane)
//   measured no faster than batches of 16.
#include "device.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace sdv {

typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const char* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p)));
}

constexpr int kProxyWaves = 4;   // waves per workgroup

// A lane's slice of a key row: VB bytes loaded non-temporally and decoded to N floats.
// 16-byte slices for f32 and bf16; fp8 rows are cut in 8-byte slices (8 channels a
// lane, sixteen lanes and so four pages a wave instead of eight), which doubles the
// number of waves of a launch.
typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));

template <int KDT, int VB>
struct ProxyVec {
  static_assert(VB == 16, "16-byte slices");
  using Raw = uint4;
  static constexpr int N = Vec16<KDT>::N;
  __device__ __forceinline__ static Raw load(const char* p) { return load_stream(p); }
  __device__ __forceinline__ static void decode(const Raw& w, float* out) { Vec16<KDT>::decode(w, out); }
};

template <>
struct ProxyVec<SDV_FP8_E4M3, 8> {
  using Raw = uint2;
  static constexpr int N = 8;
  __device__ __forceinline__ static Raw load(const char* p) {
    return __builtin_bit_cast(uint2, __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(p)));
  }
  __device__ __forceinline__ static void decode(const Raw& w, float* out) {
    fp8x2_to_f32<false>(w.x, out[0], out[1]);
    fp8x2_to_f32<true>(w.x, out[2], out[3]);
    fp8x2_to_f32<false>(w.y, out[4], out[5]);
    fp8x2_to_f32<true>(w.y, out[6], out[7]);
  }
};

template <int KDT>
constexpr int proxy_vb() { return KDT == SDV_FP8_E4M3 ? 8 : 16; }

// Value of lane l + OFF for lane l, valid where l % 16 + OFF < 16 (and for every lane
// when OFF >= 16); the halving tree reads it only in lanes whose partner is OFF above.
// Within a 16-lane row a DPP row shift does the exchange inside the vector ALU; across
// rows the LDS crossbar does.
template <int OFF>
__device__ __forceinline__ float lane_above(float v) {
  if constexpr (OFF < 16) {
    constexpr int kRowShl = 0x100;   // DPP row_shl:n, n = 1 .. 15: lane l reads lane l + n
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                              kRowShl + OFF, 0xF, 0xF, false));
  } else {
    return __shfl_xor(v, OFF, kWave);
  }
}

template <int OFF, int V>
__device__ __forceinline__ void halving_levels(float (&u)[V]) {
  if constexpr (OFF >= 1) {
#pragma unroll
    for (int e = 0; e < V; ++e) u[e] = u[e] + lane_above<OFF>(u[e]);
    halving_levels<OFF / 2, V>(u);
  }
}

// QDT: the stored query type, kept in LDS as stored (bf16 queries take half the bytes of
// float: with 8 verify tokens of 4 heads a wave stages 8 KiB instead of 16 KiB, which
// otherwise holds a CU to 10 waves where the registers allow 16).
template <int KDT, int D, int QDT>
__global__ void __launch_bounds__(64 * kProxyWaves) sdv_proxy_scores_kernel(
    const void* __restrict__ q, int32_t q_dt, const int32_t* __restrict__ qo_indptr,
    const int32_t* __restrict__ kv_len, int32_t B, int32_t max_qo_len, int32_t num_q_heads,
    int32_t G, const void* __restrict__ kbase, int64_t page_stride, int32_t num_pages,
    const int32_t* __restrict__ block_table, int32_t bt_stride, int32_t max_pages,
    float* __restrict__ scores, int32_t* dev_err) {
  using PV = ProxyVec<KDT, proxy_vb<KDT>()>;
  constexpr int V = PV::N;           // channels per lane
  constexpr int LPR = D / V;         // lanes per page
  constexpr int PPW = kWave / LPR;   // pages per wave
  constexpr int PPB = PPW * kProxyWaves;   // pages per workgroup
  constexpr int EB = elem_bytes<KDT>();
  constexpr int U = 16 * 16 / (V * EB);   // positions per unrolled step: 256 bytes a lane
  extern __shared__ float q_lds[];   // [qo][G][D] float or bf16 (QDT)
  constexpr int QEB = QDT == SDV_F32 ? 4 : 2;   // bytes per staged query channel

  // Request of this workgroup: y rotated by the page run z.  The hardware deals
  // consecutive workgroups round-robin to the eight XCDs, so without the rotation every
  // run of a request would land on the same XCDs (with four KV heads, even requests on
  // XCDs 0-3 and odd ones on 4-7) and requests of unequal length would load the XCDs
  // unevenly; rotated, a request's runs alternate between them (64 requests of
  // U[4096, 32768] bf16 tokens: 207 -> 199 us; a ragged batch 180 -> 175 us; equal-length
  // requests unchanged).
  const int r = static_cast<int>((blockIdx.y + blockIdx.z) % static_cast<uint32_t>(B));
  const int h = blockIdx.x;
  const int Hkv = gridDim.x;
  const int row0 = qo_indptr[r];
  const int qo = qo_indptr[r + 1] - row0;
  const int kv = kv_len[r];
  const bool bad_len = qo < 1 || qo > max_qo_len || kv < qo || row0 < 0 ||
                       static_cast<int64_t>(row0) + qo > static_cast<int64_t>(B) * max_qo_len;
  const bool bad_cap = !bad_len && static_cast<int64_t>(kv) > static_cast<int64_t>(max_pages) * kPage;
  if (bad_len || bad_cap) {
    if (threadIdx.x == 0 && blockIdx.z == 0 && h == 0)
      set_err(dev_err, bad_len ? SDV_DEVERR_QO_LEN : SDV_DEVERR_KV_CAPACITY);
    return;
  }
  const int n_pages_r = (kv + kPage - 1) / kPage;
  const int p_first = blockIdx.z * PPB;
  if (p_first >= n_pages_r) return;

  // This lane group's page: its block-table entry is loaded first, so that its latency
  // overlaps the query staging below.
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = lane / LPR;
  const int sub = lane - grp * LPR;
  const int p = p_first + wave * PPW + grp;
  bool active = p < n_pages_r;
  int32_t phys = 0;
  if (active) phys = block_table[static_cast<int64_t>(r) * bt_stride + p];

  // Stage this request's queries of KV head h as stored (QDT), row (t * G + g) of D
  // channels, eight channels (one 16- or 32-byte load) per item, QB items per thread in
  // flight at once.  Within a row, channel chunk k (channels 4k .. 4k + 3) sits at chunk
  // position (k % (V/4)) * LPR + k / (V/4): the e-th chunk of every lane of a page group
  // is contiguous, so the score step's reads (one chunk per lane) are free of bank
  // conflicts.
  constexpr int QB = 4;
  using QChunk = typename std::conditional<QDT == SDV_F32, float4, uint2>::type;   // 4 channels
  char* q_bytes = reinterpret_cast<char*>(q_lds);
  const int q_items = qo * G * (D / 8);
  for (int i0 = threadIdx.x; i0 < q_items; i0 += QB * blockDim.x) {
    QChunk x[QB][2];
#pragma unroll
    for (int k = 0; k < QB; ++k) {
      const int i8 = min(i0 + k * static_cast<int>(blockDim.x), q_items - 1);   // in range
      const int tg = i8 / (D / 8);
      const int c0 = (i8 - tg * (D / 8)) * 8;
      const int t = tg / G;
      const int g = tg - t * G;
      const int64_t src = (static_cast<int64_t>(row0 + t) * num_q_heads + h * G + g) * D + c0;
      if constexpr (QDT == SDV_F32) {
        const float4* s4 = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) + src);
        x[k][0] = s4[0];
        x[k][1] = s4[1];
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) + src);
        x[k][0] = make_uint2(w.x, w.y);
        x[k][1] = make_uint2(w.z, w.w);
      }
    }
#pragma unroll
    for (int k = 0; k < QB; ++k) {
      const int i8 = i0 + k * blockDim.x;
      if (i8 >= q_items) continue;
      const int tg = i8 / (D / 8);
      const int k0 = 2 * (i8 - tg * (D / 8));
      QChunk* row = reinterpret_cast<QChunk*>(q_bytes + static_cast<int64_t>(tg) * D * QEB);
      row[(k0 % (V / 4)) * LPR + k0 / (V / 4)] = x[k][0];
      row[((k0 + 1) % (V / 4)) * LPR + (k0 + 1) / (V / 4)] = x[k][1];
    }
  }
  __syncthreads();

  if (active && (phys < 0 || phys >= num_pages)) {
    set_err(dev_err, SDV_DEVERR_PAGE_RANGE);
    active = false;
  }
  if (!active) phys = 0;
  const char* kp = reinterpret_cast<const char*>(kbase) +
                   (static_cast<int64_t>(phys) * page_stride + static_cast<int64_t>(h) * kPage * D) * EB +
                   sub * proxy_vb<KDT>();
  constexpr int ROW_BYTES = D * EB;

  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  int j = 0;
  float* out_rows = scores + (static_cast<int64_t>(row0) * Hkv + h) * max_pages + p;

  // Positions of this page below token t's bound.
  auto rows_below = [&](int t) {
    const int L = active ? kv - qo + t + 1 - p * kPage : 0;
    return L < 0 ? 0 : (L > kPage ? kPage : L);
  };
  const int L_last = rows_below(qo - 1);
  // One register batch serves both the full steps and the page's last, partial stretch:
  // rows rb .. rb + U - 1 stay in w across tokens (rb < 0: w holds no such stretch), so
  // the remainder rows of every token (the last token's bound ends up to qo - 1 rows
  // further) come from one batch of loads instead of one load after another.
  typename PV::Raw w[U];
  int rb = -1;
  for (int t = 0; t < qo; ++t) {
    const int L = rows_below(t);
    // Step 1: extend the running sums to the first L positions of the page.
    for (; j + U <= L; j += U) {
      rb = -1;
      const char* rows = kp + static_cast<int64_t>(j) * ROW_BYTES;
#pragma unroll
      for (int u = 0; u < U; ++u) w[u] = PV::load(rows + u * ROW_BYTES);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[V];
        PV::decode(w[u], x);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = acc[e] + x[e];
      }
    }
    if (j < L) {
      if (rb < 0 || L > rb + U) {
        // rows j .. min(j + U, L_last) - 1; the rest of the batch repeats the last of
        // them (in bounds, never added)
        rb = j;
        const int last = (rb + U < L_last ? rb + U : L_last) - 1;
#pragma unroll
        for (int u = 0; u < U; ++u)
          w[u] = PV::load(kp + static_cast<int64_t>(rb + u < last ? rb + u : last) * ROW_BYTES);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (rb + u >= j && rb + u < L) {
          float x[V];
          PV::decode(w[u], x);
#pragma unroll
          for (int e = 0; e < V; ++e) acc[e] = acc[e] + x[e];
        }
      }
      j = L;
    }
    // Steps 2-4 for every query head of the group.
    float best = -INFINITY;
    for (int g = 0; g < G; ++g) {
      const QChunk* qv = reinterpret_cast<const QChunk*>(q_bytes + (t * G + g) * D * QEB) + sub;
      float u[V];
#pragma unroll
      for (int e4 = 0; e4 < V / 4; ++e4) {
        float4 q4;
        if constexpr (QDT == SDV_F32) {
          q4 = qv[e4 * LPR];
        } else {
          const uint2 w = qv[e4 * LPR];   // bf16 widened exactly
          q4 = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
        }
        u[4 * e4 + 0] = q4.x * acc[4 * e4 + 0];
        u[4 * e4 + 1] = q4.y * acc[4 * e4 + 1];
        u[4 * e4 + 2] = q4.z * acc[4 * e4 + 2];
        u[4 * e4 + 3] = q4.w * acc[4 * e4 + 3];
      }
      // channel c pairs with c + n/2: across lanes while n/2 >= V (lane l of the group
      // adds lane l + n/(2V), so the live lanes are the low half of the previous ones) ...
      halving_levels<LPR / 2, V>(u);
      // ... then inside the lane.
#pragma unroll
      for (int n = V; n >= 2; n >>= 1) {
#pragma unroll
        for (int e = 0; e < n / 2; ++e) u[e] = u[e] + u[e + n / 2];
      }
      best = fmaxf(best, u[0]);
    }
    if (active && sub == 0) {
      const float s = L > 0 ? best + 0.0f : -INFINITY;
      out_rows[static_cast<int64_t>(t) * Hkv * max_pages] = s;
    }
  }
}

template <int KDT, int D, int QDT>
static hipError_t launch_proxy_t(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                                 const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                 int32_t num_q_heads, const sdv_paged_kv& kv,
                                 const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
                                 float* scores, int32_t* dev_err, hipStream_t s) {
  constexpr int V = ProxyVec<KDT, proxy_vb<KDT>()>::N;
  constexpr int PPB = (kWave / (D / V)) * kProxyWaves;
  const int G = num_q_heads / kv.num_kv_heads;
  const size_t lds = static_cast<size_t>(max_qo_len) * G * D * (QDT == SDV_F32 ? 4 : 2);
  // Grid x = KV head, y = request (rotated by z in the kernel), z = run of pages:
  // workgroups are dispatched x fastest, so the runs past a request's last page (empty,
  // they exit at once) come at the end of the grid rather than between busy ones (≈ 1%
  // faster on 64 requests of U[4096, 32768] tokens).
  dim3 grid(kv.num_kv_heads, B, (max_pages + PPB - 1) / PPB);
  hipLaunchKernelGGL((sdv_proxy_scores_kernel<KDT, D, QDT>), grid, dim3(64 * kProxyWaves), lds, s, q, q_dt,
                     qo_indptr, kv_len, B, max_qo_len, num_q_heads, G, kv.k, kv.page_stride,
                     kv.num_pages, block_table, bt_stride, max_pages, scores, dev_err);
  return hipGetLastError();
}

hipError_t launch_proxy_scores(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                               const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                               int32_t num_q_heads, const sdv_paged_kv& kv,
                               const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
                               float* scores, int32_t* dev_err, hipStream_t s) {
#define SDV_PROXY_CASE(KDT, D)                                                               \
  if (kv.kv_dtype == KDT && kv.head_dim == D)                                                \
    return q_dt == SDV_F32                                                                   \
               ? launch_proxy_t<KDT, D, SDV_F32>(q, q_dt, qo_indptr, kv_len, B, max_qo_len,  \
                                                 num_q_heads, kv, block_table, max_pages,    \
                                                 bt_stride, scores, dev_err, s)              \
               : launch_proxy_t<KDT, D, SDV_BF16>(q, q_dt, qo_indptr, kv_len, B, max_qo_len, \
                                                  num_q_heads, kv, block_table, max_pages,   \
                                                  bt_stride, scores, dev_err, s);
  SDV_PROXY_CASE(SDV_F32, 64)
  SDV_PROXY_CASE(SDV_F32, 128)
  SDV_PROXY_CASE(SDV_BF16, 64)
  SDV_PROXY_CASE(SDV_BF16, 128)
  SDV_PROXY_CASE(SDV_FP8_E4M3, 64)
  SDV_PROXY_CASE(SDV_FP8_E4M3, 128)
#undef SDV_PROXY_CASE
  return hipErrorInvalidValue;
}

}  // namespace sdv
