// C ABI of the verify-attention library: argument validation (host only, before any
// HIP call), workspace layout, kernel dispatch and status reporting.
//
// The library keeps no state between calls (the last-error text is per thread and only
// reports).  Each attention entry point runs the default kernel for its arguments; the
// cross-check build (compiled with SDV_XCHECK, a separate test library) adds
// sdv_xcheck_* entry points that take the kernel family as an argument of the call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

// Kernel families (cross-check build only; the product entry points always pass
// kFamilyAuto).
constexpr int32_t kFamilyAuto = 0;      // the default kernel for the arguments
constexpr int32_t kFamilyValu = 1;      // vector-ALU kernels
constexpr int32_t kFamilyWaves = 3;     // one LDS block stream per wave
constexpr int32_t kFamilyRing = 4;      // workgroup-shared LDS block ring
constexpr int32_t kFamilyPersist = 5;   // persistent equal-range partition, per-wave body
constexpr int32_t kFamilyFlat = 6;      // persistent equal-range partition, one ring

[[maybe_unused]] bool valid_family(int32_t f) {
  return f == kFamilyAuto || f == kFamilyValu || f == kFamilyWaves || f == kFamilyRing ||
         f == kFamilyPersist || f == kFamilyFlat;
}

int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int32_t ok() {
  g_last_error.clear();
  return SDV_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SDV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool valid_dtype(int32_t dt) { return dt == SDV_F32 || dt == SDV_BF16 || dt == SDV_FP8_E4M3; }
bool valid_out_dtype(int32_t dt) { return dt == SDV_F32 || dt == SDV_BF16; }
bool valid_head_dim(int32_t d) { return d == 64 || d == 128; }
bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// q/kv element-type pairs the attention kernels implement.
bool attn_dtype_pair(int32_t q_dt, int32_t kv_dt) {
  return (q_dt == SDV_F32 && kv_dt == SDV_F32) ||
         (q_dt == SDV_BF16 && (kv_dt == SDV_BF16 || kv_dt == SDV_FP8_E4M3));
}

// Shared checks of the query-side arguments of every attention / score call.
int32_t check_query_side(const void* q, const int32_t* qo_indptr, const int32_t* kv_len,
                         int32_t B, int32_t max_qo_len, int32_t num_q_heads,
                         int32_t num_kv_heads) {
  if (B < 0) return fail(SDV_ERR_SHAPE, "batch %d < 0", B);
  if (max_qo_len < 1) return fail(SDV_ERR_SHAPE, "max_qo_len %d < 1", max_qo_len);
  if (num_kv_heads < 1) return fail(SDV_ERR_SHAPE, "num_kv_heads %d < 1", num_kv_heads);
  if (num_q_heads < 1 || num_q_heads % num_kv_heads != 0)
    return fail(SDV_ERR_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (static_cast<int64_t>(B) * num_q_heads > INT32_MAX ||
      static_cast<int64_t>(B) * max_qo_len > INT32_MAX)
    return fail(SDV_ERR_SHAPE, "batch %d too large for %d heads and max_qo_len %d", B,
                num_q_heads, max_qo_len);
  if (B > 0 && (!q || !qo_indptr || !kv_len))
    return fail(SDV_ERR_NULL_POINTER, "q, qo_indptr and kv_len must be non-null");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "q must be 16-byte aligned");
  return SDV_OK;
}

int32_t check_workspace(int32_t op, void* workspace, size_t workspace_bytes, int64_t rows_cap,
                        int32_t num_q_heads, int32_t head_dim, int32_t num_splits) {
  if (num_splits < 1 || num_splits > 4096)
    return fail(SDV_ERR_SHAPE, "num_splits %d outside [1, 4096]", num_splits);
  const size_t need = sdv_workspace_bytes(op, static_cast<int32_t>(rows_cap), num_q_heads,
                                          head_dim, num_splits);
  if (need > 0) {
    if (!workspace) return fail(SDV_ERR_WORKSPACE, "workspace of %zu bytes required, got null", need);
    if (workspace_bytes < need)
      return fail(SDV_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
      return fail(SDV_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  }
  return SDV_OK;
}

void split_workspace(void* workspace, int64_t rows_cap, int32_t num_q_heads, int32_t head_dim,
                     int32_t num_splits, float** part_o, float** part_lse) {
  if (num_splits <= 1) {
    *part_o = nullptr;
    *part_lse = nullptr;
    return;
  }
  const size_t o_bytes = align256(static_cast<size_t>(num_splits) * rows_cap * num_q_heads *
                                  head_dim * sizeof(float));
  *part_o = reinterpret_cast<float*>(workspace);
  *part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + o_bytes);
}

}  // namespace

// Device scratch of the allocation-free entry point: the split-KV partial outputs and
// log-sum-exps of verify_attention_dense_view_noalloc live here instead of in a caller
// workspace.  Each GPU holds its own copy for the life of the process.  Host code never
// uses this name as an address: the address of a device's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[SDV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the device's first call), or null
// with the failure recorded.
void* device_scratch(int32_t* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = fail(SDV_ERR_HIP, "no usable current device for the scratch buffer (%d): %s", dev,
                   hipGetErrorString(e));
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *status = fail(SDV_ERR_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *status = SDV_OK;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t sdv_workspace_bytes(int32_t op, int32_t q_rows_cap, int32_t num_q_heads,
                           int32_t head_dim, int32_t num_splits) {
  if (op != SDV_OP_VERIFY_DENSE && op != SDV_OP_VERIFY_SPARSE && op != SDV_OP_VERIFY_PAGED)
    return 0;
  if (num_splits <= 1 || q_rows_cap <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  const size_t units = static_cast<size_t>(num_splits) * q_rows_cap * num_q_heads;
  return align256(units * head_dim * sizeof(float)) + align256(units * sizeof(float));
}

const char* sdv_status_string(int32_t status) {
  switch (status) {
    case SDV_OK: return "ok";
    case SDV_ERR_NULL_POINTER: return "null pointer";
    case SDV_ERR_DTYPE: return "unsupported dtype";
    case SDV_ERR_GEOMETRY: return "unsupported geometry (native P128 draft view unavailable)";
    case SDV_ERR_SHAPE: return "bad shape";
    case SDV_ERR_WORKSPACE: return "workspace too small";
    case SDV_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* sdv_last_error(void) { return g_last_error.c_str(); }

int32_t kv_subpage_view_init(const sdv_subpage_geom* geom, const int32_t* block_table,
                             int32_t B, int32_t max_blocks, int32_t bt_stride,
                             int32_t* sub_offsets, sdv_subpage_view* view_out,
                             int32_t* dev_err, hipStream_t stream) {
  if (!geom || !view_out) return fail(SDV_ERR_NULL_POINTER, "geom and view_out must be non-null");
  const sdv_subpage_geom& g = *geom;
  const char* why = nullptr;
  char buf[160];
  if (g.phys_page != SDV_PHYS_PAGE) {
    snprintf(buf, sizeof buf, "physical page is %d tokens, the view needs 128", g.phys_page);
    why = buf;
  } else if (g.sub_page != SDV_SUB_PAGE) {
    snprintf(buf, sizeof buf, "sub-page is %d tokens, the view needs 32", g.sub_page);
    why = buf;
  } else if (g.num_layers != 1) {
    snprintf(buf, sizeof buf, "view spans %d layers, it must be single-layer", g.num_layers);
    why = buf;
  } else if (g.kv_offset != 1) {
    snprintf(buf, sizeof buf, "kv_offset is %d, V must be the page after K (1)", g.kv_offset);
    why = buf;
  } else if (g.slot_stride < 2) {
    snprintf(buf, sizeof buf, "slot stride %d cannot hold a K and a V page", g.slot_stride);
    why = buf;
  } else if (g.num_kv_heads < 1) {
    snprintf(buf, sizeof buf, "num_kv_heads %d < 1", g.num_kv_heads);
    why = buf;
  } else if (!valid_head_dim(g.head_dim)) {
    snprintf(buf, sizeof buf, "head_dim %d (supported: 64, 128)", g.head_dim);
    why = buf;
  } else if (g.num_slots < 1 ||
             static_cast<int64_t>(g.num_slots) * g.slot_stride * 4 >= (1ll << 31)) {
    snprintf(buf, sizeof buf, "num_slots %d with stride %d exceeds the 32-bit P32 index range",
             g.num_slots, g.slot_stride);
    why = buf;
  }
  if (why) return fail(SDV_ERR_GEOMETRY, "native P128 draft view unavailable: %s", why);
  if (!valid_dtype(g.kv_dtype)) return fail(SDV_ERR_DTYPE, "kv_dtype %d", g.kv_dtype);
  if (!valid_scale(g.k_scale) || !valid_scale(g.v_scale))
    return fail(SDV_ERR_SHAPE, "k_scale and v_scale must be finite and > 0");
  if (!g.k_root) return fail(SDV_ERR_NULL_POINTER, "k_root must be non-null");
  if (reinterpret_cast<uintptr_t>(g.k_root) % 16 != 0)
    return fail(SDV_ERR_GEOMETRY, "native P128 draft view unavailable: k_root not 16-byte aligned");
  if (B < 0 || max_blocks < 0 || bt_stride < max_blocks)
    return fail(SDV_ERR_SHAPE, "B %d, max_blocks %d, bt_stride %d", B, max_blocks, bt_stride);
  if (B > 0 && max_blocks > 0 && (!block_table || !sub_offsets))
    return fail(SDV_ERR_NULL_POINTER, "block_table and sub_offsets must be non-null");

  view_out->k_root = g.k_root;
  view_out->kv_dtype = g.kv_dtype;
  view_out->num_kv_heads = g.num_kv_heads;
  view_out->head_dim = g.head_dim;
  view_out->index_scale = g.slot_stride;
  view_out->num_slots = g.num_slots;
  view_out->k_scale = g.k_scale;
  view_out->v_scale = g.v_scale;
  // P32 pages from the root up to and including the last slot's V page.
  view_out->num_sub_pages = 4ll * ((static_cast<int64_t>(g.num_slots) - 1) * g.slot_stride + 2);
  if (B == 0 || max_blocks == 0) return ok();
  return hip_status(sdv::launch_subpage_offsets(block_table, B, max_blocks, bt_stride,
                                                g.slot_stride, g.num_slots, sub_offsets,
                                                dev_err, stream),
                    "kv_subpage_view_init launch");
}

}  // extern "C"

// Dense verify attention through the P32 view: block indices from sub_offsets, or (null)
// from block_table as the view defines them.
static int32_t dense_attention(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                               const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                               int32_t num_q_heads, const sdv_subpage_view* view,
                               const int32_t* sub_offsets, int32_t max_sub_pages,
                               const int32_t* block_table, int32_t bt_stride,
                               float softmax_scale, int32_t num_splits, void* workspace,
                               size_t workspace_bytes, void* out, int32_t out_dt,
                               int32_t* dev_err, hipStream_t stream, const char* name,
                               int32_t fam) {
  if (!view) return fail(SDV_ERR_NULL_POINTER, "view must be non-null");
  const sdv_subpage_view& v = *view;
  int32_t st = check_query_side(q, qo_indptr, kv_len, B, max_qo_len, num_q_heads, v.num_kv_heads);
  if (st) return st;
  if (!attn_dtype_pair(q_dt, v.kv_dtype))
    return fail(SDV_ERR_DTYPE, "q dtype %d with kv dtype %d", q_dt, v.kv_dtype);
  if (!valid_out_dtype(out_dt)) return fail(SDV_ERR_DTYPE, "out dtype %d", out_dt);
  if (!valid_head_dim(v.head_dim)) return fail(SDV_ERR_SHAPE, "head_dim %d", v.head_dim);
  const int32_t G = num_q_heads / v.num_kv_heads;
  if (static_cast<int64_t>(G) * max_qo_len > 64)
    return fail(SDV_ERR_SHAPE, "group %d x max_qo_len %d exceeds 64 query rows", G, max_qo_len);
  if (max_sub_pages < 1) return fail(SDV_ERR_SHAPE, "max_sub_pages %d < 1", max_sub_pages);
  if (num_splits >= 1 &&
      (static_cast<int64_t>(max_sub_pages) + num_splits - 1) / num_splits > sdv::kMaxSplitBlocks)
    return fail(SDV_ERR_SHAPE, "num_splits %d too small: each split may hold at most %d "
                "32-token blocks of the %d-sub-page capacity", num_splits, sdv::kMaxSplitBlocks,
                max_sub_pages);
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(SDV_ERR_SHAPE, "softmax_scale must be finite and > 0");
  if (!valid_scale(v.k_scale) || !valid_scale(v.v_scale) || !v.k_root || v.num_sub_pages < 8)
    return fail(SDV_ERR_GEOMETRY, "native P128 draft view unavailable: view not initialised");
  const int64_t rows_cap = static_cast<int64_t>(B) * max_qo_len;
  if (rows_cap > (1ll << 30)) return fail(SDV_ERR_SHAPE, "too many query rows");
  st = check_workspace(SDV_OP_VERIFY_DENSE, workspace, workspace_bytes, rows_cap, num_q_heads,
                       v.head_dim, num_splits);
  if (st) return st;
  if (B > 0 && ((!sub_offsets && !block_table) || !out))
    return fail(SDV_ERR_NULL_POINTER, "%s and out must be non-null",
                block_table ? "block_table" : "sub_offsets");
  if (reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "out must be 16-byte aligned");
  if (B == 0) return ok();

  sdv::AttnArgs a{};
  a.q = q; a.q_dt = q_dt; a.qo_indptr = qo_indptr; a.kv_len = kv_len; a.B = B;
  a.max_qo_len = max_qo_len; a.num_q_heads = num_q_heads; a.num_kv_heads = v.num_kv_heads;
  a.head_dim = v.head_dim; a.kv_dt = v.kv_dtype; a.k_scale = v.k_scale; a.v_scale = v.v_scale;
  a.softmax_scale = softmax_scale; a.num_splits = num_splits; a.out = out; a.out_dt = out_dt;
  a.dev_err = dev_err;
  split_workspace(workspace, rows_cap, num_q_heads, v.head_dim, num_splits, &a.part_o, &a.part_lse);
  sdv::DenseSource src{v.k_root, sub_offsets, max_sub_pages, v.num_sub_pages,
                       sub_offsets ? nullptr : block_table, bt_stride, v.index_scale, v.num_slots};
  // Default: the per-split ring while the (request, KV head) pairs fit the GPU's resident
  // workgroups a few times over; with more pairs than twice the compute units (the ring
  // holds two workgroups per CU), the per-split grid queues and its imbalance compounds,
  // so the flat persistent kernel, which gives every workgroup an equal block range, takes
  // over (measured on the ragged 256-request batch: 378 against 432-458 us).
  const bool many_pairs =
      static_cast<int64_t>(B) * v.num_kv_heads >= 2ll * std::max(1, sdv::device_cu_count());
  const bool persist_ok = sdv::persist_supported(a, max_sub_pages);
  hipError_t e;
  if (fam == kFamilyValu || !sdv::mfma_supported(a)) e = sdv::launch_attn_dense_valu(a, src, stream);
  else if (fam == kFamilyWaves) e = sdv::launch_attn_dense_waves(a, src, stream);
  else if (fam == kFamilyPersist && persist_ok) e = sdv::launch_attn_dense_persist(a, src, stream);
  else if ((fam == kFamilyFlat || (fam == kFamilyAuto && many_pairs)) && persist_ok)
    e = sdv::launch_attn_dense_flat(a, src, stream);
  else e = sdv::launch_attn_dense_stream(a, src, stream);   // the ring, and the persistent
                                                            // kernels where they do not apply
  if (e != hipSuccess) return hip_status(e, name);
  if (num_splits > 1) {
    e = sdv::launch_combine(a.part_o, a.part_lse, num_splits, static_cast<int32_t>(rows_cap),
                            qo_indptr, qo_indptr + B, num_q_heads, v.head_dim, out, out_dt,
                            nullptr, stream);
    if (e != hipSuccess) return hip_status(e, name);
  }
  return ok();
}

extern "C" {

}  // extern "C"

static int32_t dense_offsets_call(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                                  const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                  int32_t num_q_heads, const sdv_subpage_view* view,
                                  const int32_t* sub_offsets, int32_t max_sub_pages,
                                  float softmax_scale, int32_t num_splits, void* workspace,
                                  size_t workspace_bytes, void* out, int32_t out_dt,
                                  int32_t* dev_err, hipStream_t stream, int32_t fam) {
  if (B > 0 && !sub_offsets) return fail(SDV_ERR_NULL_POINTER, "sub_offsets must be non-null");
  return dense_attention(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, view,
                         sub_offsets, max_sub_pages, nullptr, 0, softmax_scale, num_splits,
                         workspace, workspace_bytes, out, out_dt, dev_err, stream,
                         "verify_attention_dense launch", fam);
}

static int32_t dense_view_call(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                               const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                               int32_t num_q_heads, const sdv_subpage_view* view,
                               const int32_t* block_table, int32_t max_blocks,
                               int32_t bt_stride, float softmax_scale, int32_t num_splits,
                               void* workspace, size_t workspace_bytes, void* out,
                               int32_t out_dt, int32_t* dev_err, hipStream_t stream,
                               int32_t fam) {
  if (max_blocks < 1 || bt_stride < max_blocks)
    return fail(SDV_ERR_SHAPE, "max_blocks %d, bt_stride %d", max_blocks, bt_stride);
  if (static_cast<int64_t>(max_blocks) * 4 > INT32_MAX / 32)
    return fail(SDV_ERR_SHAPE, "max_blocks %d too large", max_blocks);
  if (B > 0 && !block_table) return fail(SDV_ERR_NULL_POINTER, "block_table must be non-null");
  return dense_attention(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, view, nullptr,
                         4 * max_blocks, block_table, bt_stride, softmax_scale, num_splits,
                         workspace, workspace_bytes, out, out_dt, dev_err, stream,
                         "verify_attention_dense_view launch", fam);
}

extern "C" {

int32_t verify_attention_dense(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                               const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                               int32_t num_q_heads, const sdv_subpage_view* view,
                               const int32_t* sub_offsets, int32_t max_sub_pages,
                               float softmax_scale, int32_t num_splits, void* workspace,
                               size_t workspace_bytes, void* out, int32_t out_dt,
                               int32_t* dev_err, hipStream_t stream) {
  return dense_offsets_call(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, view,
                            sub_offsets, max_sub_pages, softmax_scale, num_splits, workspace,
                            workspace_bytes, out, out_dt, dev_err, stream, kFamilyAuto);
}

int32_t verify_attention_dense_view(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                                    const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                    int32_t num_q_heads, const sdv_subpage_view* view,
                                    const int32_t* block_table, int32_t max_blocks,
                                    int32_t bt_stride, float softmax_scale, int32_t num_splits,
                                    void* workspace, size_t workspace_bytes, void* out,
                                    int32_t out_dt, int32_t* dev_err, hipStream_t stream) {
  return dense_view_call(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, view,
                         block_table, max_blocks, bt_stride, softmax_scale, num_splits,
                         workspace, workspace_bytes, out, out_dt, dev_err, stream, kFamilyAuto);
}

int32_t verify_attention_dense_view_noalloc(const void* q, int32_t q_dt,
                                            const int32_t* qo_indptr, const int32_t* kv_len,
                                            int32_t B, int32_t max_qo_len, int32_t num_q_heads,
                                            const sdv_subpage_view* view,
                                            const int32_t* block_table, int32_t max_blocks,
                                            int32_t bt_stride, float softmax_scale,
                                            int32_t num_splits, void* out, int32_t out_dt,
                                            int32_t* dev_err, hipStream_t stream) {
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (B > 0 && num_splits > 1 && view && view->num_kv_heads >= 1 &&
      num_q_heads % view->num_kv_heads == 0) {
    const size_t need = sdv_workspace_bytes(SDV_OP_VERIFY_DENSE,
                                            static_cast<int32_t>(std::min<int64_t>(
                                                static_cast<int64_t>(B) * max_qo_len, INT32_MAX)),
                                            num_q_heads, view->head_dim, num_splits);
    if (need > SDV_NOALLOC_SCRATCH_BYTES)
      return fail(SDV_ERR_WORKSPACE, "the call needs %zu bytes of split-KV scratch, the "
                  "allocation-free entry point holds %zu: use fewer splits or rows, or "
                  "verify_attention_dense_view with a workspace", need,
                  static_cast<size_t>(SDV_NOALLOC_SCRATCH_BYTES));
    if (need > 0) {
      int32_t st = SDV_OK;
      ws = device_scratch(&st);
      if (!ws) return st;
      ws_bytes = SDV_NOALLOC_SCRATCH_BYTES;
    }
  }
  return dense_view_call(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, view,
                         block_table, max_blocks, bt_stride, softmax_scale, num_splits, ws,
                         ws_bytes, out, out_dt, dev_err, stream, kFamilyAuto);
}

static int32_t check_paged_kv(const sdv_paged_kv* kv) {
  if (!kv) return fail(SDV_ERR_NULL_POINTER, "kv must be non-null");
  if (kv->page_size != SDV_PHYS_PAGE)
    return fail(SDV_ERR_GEOMETRY, "page_size %d (supported: 128)", kv->page_size);
  if (kv->num_kv_heads < 1) return fail(SDV_ERR_SHAPE, "num_kv_heads %d", kv->num_kv_heads);
  if (!valid_head_dim(kv->head_dim)) return fail(SDV_ERR_SHAPE, "head_dim %d", kv->head_dim);
  if (!valid_dtype(kv->kv_dtype)) return fail(SDV_ERR_DTYPE, "kv dtype %d", kv->kv_dtype);
  if (kv->num_pages < 1) return fail(SDV_ERR_SHAPE, "num_pages %d", kv->num_pages);
  if (kv->page_stride < static_cast<int64_t>(kv->num_kv_heads) * SDV_PHYS_PAGE * kv->head_dim)
    return fail(SDV_ERR_SHAPE, "page_stride %lld smaller than one page",
                static_cast<long long>(kv->page_stride));
  const int eb = kv->kv_dtype == SDV_F32 ? 4 : (kv->kv_dtype == SDV_BF16 ? 2 : 1);
  if ((kv->page_stride * eb) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "page stride must be a multiple of 16 bytes");
  if (!kv->k || !kv->v) return fail(SDV_ERR_NULL_POINTER, "kv.k and kv.v must be non-null");
  if ((reinterpret_cast<uintptr_t>(kv->k) | reinterpret_cast<uintptr_t>(kv->v)) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "K and V pools must be 16-byte aligned");
  if (!valid_scale(kv->k_scale) || !valid_scale(kv->v_scale))
    return fail(SDV_ERR_SHAPE, "k_scale and v_scale must be finite and > 0");
  return SDV_OK;
}

int32_t proxy_page_scores(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                          const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                          int32_t num_q_heads, const sdv_paged_kv* kv,
                          const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
                          float* scores, int32_t* dev_err, hipStream_t stream) {
  int32_t st = check_paged_kv(kv);
  if (st) return st;
  st = check_query_side(q, qo_indptr, kv_len, B, max_qo_len, num_q_heads, kv->num_kv_heads);
  if (st) return st;
  if (q_dt != SDV_F32 && q_dt != SDV_BF16) return fail(SDV_ERR_DTYPE, "q dtype %d", q_dt);
  const int32_t G = num_q_heads / kv->num_kv_heads;
  if (static_cast<int64_t>(max_qo_len) * G * kv->head_dim > 8192)
    return fail(SDV_ERR_SHAPE, "max_qo_len x group x head_dim exceeds 8192");
  if (max_pages < 1 || bt_stride < max_pages)
    return fail(SDV_ERR_SHAPE, "max_pages %d, bt_stride %d", max_pages, bt_stride);
  // launch grid: y = request, z = run of pages (each at most 65535; a run holds at least
  // two pages: four or eight but for f32 keys of head_dim 128)
  if (B > 65535 || max_pages > 2 * 65535)
    return fail(SDV_ERR_SHAPE, "batch %d (<= 65535) or max_pages %d (<= 131070)", B, max_pages);
  if (B > 0 && (!block_table || !scores))
    return fail(SDV_ERR_NULL_POINTER, "block_table and scores must be non-null");
  if (B == 0) return ok();
  return hip_status(sdv::launch_proxy_scores(q, q_dt, qo_indptr, kv_len, B, max_qo_len,
                                             num_q_heads, *kv, block_table, max_pages, bt_stride,
                                             scores, dev_err, stream),
                    "proxy_page_scores launch");
}

int32_t ladder_topk_pages(const float* scores, const int32_t* qo_indptr, const int32_t* kv_len,
                          int32_t B, int32_t max_qo_len, int32_t num_kv_heads, int32_t max_pages,
                          int32_t page_size, int32_t top_k, int32_t* topk_idx,
                          int32_t* topk_cnt, int32_t* dev_err, hipStream_t stream) {
  if (page_size != SDV_PHYS_PAGE)
    return fail(SDV_ERR_GEOMETRY, "page_size %d (supported: 128)", page_size);
  if (B < 0 || max_qo_len < 1 || num_kv_heads < 1)
    return fail(SDV_ERR_SHAPE, "B %d, max_qo_len %d, num_kv_heads %d", B, max_qo_len, num_kv_heads);
  if (top_k < 1 || top_k > 1024) return fail(SDV_ERR_SHAPE, "top_k %d outside [1, 1024]", top_k);
  if (max_pages < 1 || max_pages > 4096)
    return fail(SDV_ERR_SHAPE, "max_pages %d outside [1, 4096]", max_pages);
  if (B > 65535) return fail(SDV_ERR_SHAPE, "batch %d (<= 65535: one launch-grid row each)", B);
  if (B > 0 && (!scores || !qo_indptr || !kv_len || !topk_idx))
    return fail(SDV_ERR_NULL_POINTER, "scores, qo_indptr, kv_len and topk_idx must be non-null");
  if (B == 0) return ok();
  return hip_status(sdv::launch_topk(scores, qo_indptr, kv_len, B, max_qo_len, num_kv_heads,
                                     max_pages, top_k, topk_idx, topk_cnt, dev_err, stream),
                    "ladder_topk_pages launch");
}

// Shared checks of the staging calls' new rows and lengths.
static int32_t check_stage_rows(const void* k_new, const void* v_new, int32_t new_dt,
                                int32_t kv_dt, const int32_t* qo_indptr, const int32_t* kv_len,
                                int32_t B, int32_t max_qo_len) {
  if (B < 0) return fail(SDV_ERR_SHAPE, "batch %d < 0", B);
  if (max_qo_len < 1) return fail(SDV_ERR_SHAPE, "max_qo_len %d < 1", max_qo_len);
  if (static_cast<int64_t>(B) * max_qo_len > INT32_MAX)
    return fail(SDV_ERR_SHAPE, "batch %d x max_qo_len %d too large", B, max_qo_len);
  if (new_dt != kv_dt)
    return fail(SDV_ERR_DTYPE, "new rows dtype %d differs from the cache dtype %d (rows are "
                "copied as stored)", new_dt, kv_dt);
  if (B > 0 && (!k_new || !v_new || !qo_indptr || !kv_len))
    return fail(SDV_ERR_NULL_POINTER, "k_new, v_new, qo_indptr and kv_len must be non-null");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "k_new and v_new must be 16-byte aligned");
  return SDV_OK;
}

int32_t stage_verify_kv_paged(const void* k_new, const void* v_new, int32_t new_dt,
                              const int32_t* qo_indptr, const int32_t* kv_len, int32_t B,
                              int32_t max_qo_len, const sdv_paged_kv* kv,
                              const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
                              int32_t* dev_err, hipStream_t stream) {
  int32_t st = check_paged_kv(kv);
  if (st) return st;
  st = check_stage_rows(k_new, v_new, new_dt, kv->kv_dtype, qo_indptr, kv_len, B, max_qo_len);
  if (st) return st;
  if (max_pages < 1 || max_pages > (1 << 20) || bt_stride < max_pages)
    return fail(SDV_ERR_SHAPE, "max_pages %d (<= 2^20), bt_stride %d", max_pages, bt_stride);
  if (B > 0 && !block_table) return fail(SDV_ERR_NULL_POINTER, "block_table must be non-null");
  if (B == 0) return ok();
  return hip_status(sdv::launch_stage_paged(k_new, v_new, qo_indptr, kv_len, B, max_qo_len, *kv,
                                            block_table, max_pages, bt_stride, dev_err, stream),
                    "stage_verify_kv_paged launch");
}

int32_t stage_verify_kv_view(const void* k_new, const void* v_new, int32_t new_dt,
                             const int32_t* qo_indptr, const int32_t* kv_len, int32_t B,
                             int32_t max_qo_len, const sdv_subpage_view* view,
                             const int32_t* sub_offsets, int32_t max_sub_pages,
                             int32_t* dev_err, hipStream_t stream) {
  if (!view) return fail(SDV_ERR_NULL_POINTER, "view must be non-null");
  if (!view->k_root || view->num_sub_pages < 8 || !valid_head_dim(view->head_dim) ||
      view->num_kv_heads < 1 || !valid_dtype(view->kv_dtype))
    return fail(SDV_ERR_GEOMETRY, "native P128 draft view unavailable: view not initialised");
  int32_t st = check_stage_rows(k_new, v_new, new_dt, view->kv_dtype, qo_indptr, kv_len, B,
                                max_qo_len);
  if (st) return st;
  if (max_sub_pages < 1) return fail(SDV_ERR_SHAPE, "max_sub_pages %d < 1", max_sub_pages);
  if (B > 0 && !sub_offsets) return fail(SDV_ERR_NULL_POINTER, "sub_offsets must be non-null");
  if (B == 0) return ok();
  return hip_status(sdv::launch_stage_view(k_new, v_new, qo_indptr, kv_len, B, max_qo_len, *view,
                                           sub_offsets, max_sub_pages, dev_err, stream),
                    "stage_verify_kv_view launch");
}

int32_t hnd_head_slice_descriptors(int32_t token_groups, int32_t src_heads,
                                   int32_t src_head_begin, int32_t dst_heads,
                                   int32_t dst_head_begin, int32_t num_heads,
                                   int32_t head_dim, int32_t kv_dtype, int32_t page_tokens,
                                   const int64_t* src_page_offsets,
                                   const int64_t* dst_page_offsets, int32_t num_pages,
                                   sdv_copy_desc* out, int32_t capacity, int32_t* count_out) {
  if (!valid_dtype(kv_dtype)) return fail(SDV_ERR_DTYPE, "kv dtype %d", kv_dtype);
  if (token_groups < 1 || page_tokens < 1 || page_tokens % token_groups != 0)
    return fail(SDV_ERR_SHAPE, "page_tokens %d is not a multiple of token_groups %d",
                page_tokens, token_groups);
  if (head_dim < 1 || num_heads < 1 || src_heads < 1 || dst_heads < 1 || src_head_begin < 0 ||
      dst_head_begin < 0 || src_head_begin + num_heads > src_heads ||
      dst_head_begin + num_heads > dst_heads)
    return fail(SDV_ERR_SHAPE, "heads [%d, +%d) of %d to [%d, +%d) of %d", src_head_begin,
                num_heads, src_heads, dst_head_begin, num_heads, dst_heads);
  if (num_pages < 0) return fail(SDV_ERR_SHAPE, "num_pages %d < 0", num_pages);
  if (!count_out) return fail(SDV_ERR_NULL_POINTER, "count_out must be non-null");
  const int64_t need = static_cast<int64_t>(num_pages) * token_groups;
  *count_out = static_cast<int32_t>(need > INT32_MAX ? INT32_MAX : need);
  if (need > capacity) return fail(SDV_ERR_SHAPE, "capacity %d < %lld descriptors", capacity,
                                   static_cast<long long>(need));
  if (num_pages > 0 && (!src_page_offsets || !dst_page_offsets || !out))
    return fail(SDV_ERR_NULL_POINTER, "page offsets and out must be non-null");
  const int64_t row = static_cast<int64_t>(page_tokens / token_groups) * head_dim *
                      sdv::elem_bytes_of(kv_dtype);   // one head in one group
  int64_t k = 0;
  for (int32_t i = 0; i < num_pages; ++i)
    for (int32_t g = 0; g < token_groups; ++g, ++k) {
      out[k].src_offset = src_page_offsets[i] + (static_cast<int64_t>(g) * src_heads + src_head_begin) * row;
      out[k].dst_offset = dst_page_offsets[i] + (static_cast<int64_t>(g) * dst_heads + dst_head_begin) * row;
      out[k].bytes = num_heads * row;
    }
  return ok();
}

int32_t copy_descriptors(const void* src_base, size_t src_bytes, void* dst_base,
                         size_t dst_bytes, const sdv_copy_desc* descs, int32_t num_descs,
                         int32_t* dev_err, hipStream_t stream) {
  if (num_descs < 0) return fail(SDV_ERR_SHAPE, "num_descs %d < 0", num_descs);
  if (num_descs == 0) return ok();
  if (!src_base || !dst_base || !descs)
    return fail(SDV_ERR_NULL_POINTER, "src_base, dst_base and descs must be non-null");
  if ((reinterpret_cast<uintptr_t>(src_base) | reinterpret_cast<uintptr_t>(dst_base)) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "src_base and dst_base must be 16-byte aligned");
  return hip_status(sdv::launch_copy_descriptors(src_base, src_bytes, dst_base, dst_bytes, descs,
                                                 num_descs, dev_err, stream),
                    "copy_descriptors launch");
}

size_t sdv_greedy_accept_workspace_bytes(int32_t B, int32_t max_qo_len, int32_t vocab,
                                     int32_t logits_dt) {
  if (B < 0 || max_qo_len < 1 || vocab < 1 || (logits_dt != SDV_F32 && logits_dt != SDV_BF16))
    return 0;
  return static_cast<size_t>(B) * static_cast<size_t>(max_qo_len) *
         static_cast<size_t>(sdv::greedy_accept_parts(vocab, logits_dt)) * 8u;
}

int32_t greedy_accept(const void* logits, int32_t logits_dt, int32_t vocab,
                      const int32_t* tokens, const int32_t* qo_indptr, const int32_t* kv_len,
                      int32_t B, int32_t max_qo_len, void* workspace, size_t workspace_bytes,
                      int32_t* targets_out, int32_t* accept_out, int32_t* emitted_out,
                      int32_t* new_kv_len_out, int32_t* dev_err, hipStream_t stream) {
  if (logits_dt != SDV_F32 && logits_dt != SDV_BF16)
    return fail(SDV_ERR_DTYPE, "logits dtype %d (supported: F32, BF16)", logits_dt);
  const int per = logits_dt == SDV_F32 ? 4 : 8;
  if (vocab < 1 || vocab % per != 0)
    return fail(SDV_ERR_SHAPE, "vocab %d must be a positive multiple of %d", vocab, per);
  if (B < 0 || max_qo_len < 1 || static_cast<int64_t>(B) * max_qo_len > INT32_MAX)
    return fail(SDV_ERR_SHAPE, "B %d, max_qo_len %d", B, max_qo_len);
  const int64_t wgs = static_cast<int64_t>(B) * max_qo_len * sdv::greedy_accept_parts(vocab, logits_dt);
  if (wgs > INT32_MAX)
    return fail(SDV_ERR_SHAPE, "B * max_qo_len * ceil(vocab / %d) = %lld exceeds the grid limit",
                per * 1024, static_cast<long long>(wgs));
  if (B == 0) return ok();
  if (!logits || !tokens || !qo_indptr || !kv_len || !workspace || !targets_out || !accept_out ||
      !emitted_out || !new_kv_len_out)
    return fail(SDV_ERR_NULL_POINTER, "every array argument but dev_err must be non-null");
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "logits must be 16-byte aligned");
  const size_t need = sdv_greedy_accept_workspace_bytes(B, max_qo_len, vocab, logits_dt);
  if (workspace_bytes < need)
    return fail(SDV_ERR_WORKSPACE, "workspace holds %zu bytes, the call needs %zu",
                workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 8 != 0)
    return fail(SDV_ERR_SHAPE, "workspace must be 8-byte aligned");
  return hip_status(sdv::launch_greedy_accept(logits, logits_dt, vocab, tokens, qo_indptr, kv_len,
                                              B, max_qo_len, workspace, targets_out, accept_out,
                                              emitted_out, new_kv_len_out, dev_err, stream),
                    "greedy_accept launch");
}

}  // extern "C"

static int32_t paged_call(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                          const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                          int32_t num_q_heads, const sdv_paged_kv* kv,
                          const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
                          float softmax_scale, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, void* out, int32_t out_dt, int32_t* dev_err,
                          hipStream_t stream, int32_t fam) {
  int32_t st = check_paged_kv(kv);
  if (st) return st;
  st = check_query_side(q, qo_indptr, kv_len, B, max_qo_len, num_q_heads, kv->num_kv_heads);
  if (st) return st;
  if (q_dt != SDV_BF16 || (kv->kv_dtype != SDV_BF16 && kv->kv_dtype != SDV_FP8_E4M3))
    return fail(SDV_ERR_DTYPE, "q dtype %d with kv dtype %d (supported: BF16 q, BF16/FP8 K/V)",
                q_dt, kv->kv_dtype);
  if (!valid_out_dtype(out_dt)) return fail(SDV_ERR_DTYPE, "out dtype %d", out_dt);
  const int32_t G = num_q_heads / kv->num_kv_heads;
  if (static_cast<int64_t>(G) * max_qo_len > 64)
    return fail(SDV_ERR_SHAPE, "group %d x max_qo_len %d exceeds 64 query rows", G, max_qo_len);
  if (max_qo_len > 32) return fail(SDV_ERR_SHAPE, "max_qo_len %d > 32", max_qo_len);
  if (max_pages < 1 || max_pages > (1 << 20) || bt_stride < max_pages)
    return fail(SDV_ERR_SHAPE, "max_pages %d (<= 2^20), bt_stride %d", max_pages, bt_stride);
  if (num_splits < 1 || (4ll * max_pages + num_splits - 1) / num_splits > sdv::kMaxSplitBlocks)
    return fail(SDV_ERR_SHAPE, "num_splits %d too small: each split may hold at most %d "
                "32-token blocks of the %d-page capacity", num_splits,
                sdv::kMaxSplitBlocks, max_pages);
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(SDV_ERR_SHAPE, "softmax_scale must be finite and > 0");
  const int64_t rows_cap = static_cast<int64_t>(B) * max_qo_len;
  if (rows_cap > (1ll << 30)) return fail(SDV_ERR_SHAPE, "too many query rows");
  st = check_workspace(SDV_OP_VERIFY_PAGED, workspace, workspace_bytes, rows_cap, num_q_heads,
                       kv->head_dim, num_splits);
  if (st) return st;
  if (B > 0 && (!block_table || !out))
    return fail(SDV_ERR_NULL_POINTER, "block_table and out must be non-null");
  if (reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "out must be 16-byte aligned");
  if (B == 0) return ok();

  sdv::AttnArgs a{};
  a.q = q; a.q_dt = q_dt; a.qo_indptr = qo_indptr; a.kv_len = kv_len; a.B = B;
  a.max_qo_len = max_qo_len; a.num_q_heads = num_q_heads; a.num_kv_heads = kv->num_kv_heads;
  a.head_dim = kv->head_dim; a.kv_dt = kv->kv_dtype; a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale; a.softmax_scale = softmax_scale; a.num_splits = num_splits;
  a.out = out; a.out_dt = out_dt; a.dev_err = dev_err;
  split_workspace(workspace, rows_cap, num_q_heads, kv->head_dim, num_splits, &a.part_o, &a.part_lse);
  sdv::SparseSource src{kv->k, kv->v, kv->page_stride, kv->num_pages, block_table, bt_stride,
                        max_pages, nullptr, 0};
  hipError_t e;
  if (fam == kFamilyRing) e = sdv::launch_attn_paged_stream(a, src, stream);
  else if (fam == kFamilyWaves || !sdv::persist_supported(a, 4ll * max_pages))
    e = sdv::launch_attn_paged_waves(a, src, stream);
  else if (fam == kFamilyFlat) e = sdv::launch_attn_paged_flat(a, src, stream);
  else e = sdv::launch_attn_paged_persist(a, src, stream);   // automatic and persistent
  if (e != hipSuccess) return hip_status(e, "verify_attention_paged launch");
  if (num_splits > 1) {
    e = sdv::launch_combine(a.part_o, a.part_lse, num_splits, static_cast<int32_t>(rows_cap),
                            qo_indptr, qo_indptr + B, num_q_heads, kv->head_dim, out, out_dt,
                            nullptr, stream);
    if (e != hipSuccess) return hip_status(e, "verify_attention_paged combine launch");
  }
  return ok();
}

extern "C" {

int32_t verify_attention_paged(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                               const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                               int32_t num_q_heads, const sdv_paged_kv* kv,
                               const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
                               float softmax_scale, int32_t num_splits, void* workspace,
                               size_t workspace_bytes, void* out, int32_t out_dt,
                               int32_t* dev_err, hipStream_t stream) {
  return paged_call(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, kv, block_table,
                    max_pages, bt_stride, softmax_scale, num_splits, workspace, workspace_bytes,
                    out, out_dt, dev_err, stream, kFamilyAuto);
}

}  // extern "C"

// Sparse verify attention over the pages in topk_idx, or (scores non-null) over the
// ladder top-k of scores selected inside the attention kernels.
static int32_t sparse_attention(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                                const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                int32_t num_q_heads, const sdv_paged_kv* kv,
                                const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
                                const int32_t* topk_idx, const float* scores, int32_t* topk_out,
                                int32_t* cnt_out, int32_t top_k, float softmax_scale,
                                int32_t num_splits, void* workspace, size_t workspace_bytes,
                                void* out, int32_t out_dt, int32_t* dev_err, hipStream_t stream,
                                const char* name, int32_t fam) {
  int32_t st = check_paged_kv(kv);
  if (st) return st;
  st = check_query_side(q, qo_indptr, kv_len, B, max_qo_len, num_q_heads, kv->num_kv_heads);
  if (st) return st;
  if (!attn_dtype_pair(q_dt, kv->kv_dtype))
    return fail(SDV_ERR_DTYPE, "q dtype %d with kv dtype %d", q_dt, kv->kv_dtype);
  if (!valid_out_dtype(out_dt)) return fail(SDV_ERR_DTYPE, "out dtype %d", out_dt);
  const int32_t G = num_q_heads / kv->num_kv_heads;
  if (static_cast<int64_t>(G) * max_qo_len > 64)
    return fail(SDV_ERR_SHAPE, "group %d x max_qo_len %d exceeds 64 query rows", G, max_qo_len);
  if (max_qo_len > 32) return fail(SDV_ERR_SHAPE, "max_qo_len %d > 32", max_qo_len);
  if (top_k < 1 || static_cast<int64_t>(top_k) * max_qo_len > 512)
    return fail(SDV_ERR_SHAPE, "top_k %d x max_qo_len %d outside [1, 512]", top_k, max_qo_len);
  if (max_pages < 1 || max_pages > 16384 || bt_stride < max_pages)
    return fail(SDV_ERR_SHAPE, "max_pages %d (<= 16384), bt_stride %d", max_pages, bt_stride);
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(SDV_ERR_SHAPE, "softmax_scale must be finite and > 0");
  const int64_t rows_cap = static_cast<int64_t>(B) * max_qo_len;
  if (rows_cap > (1ll << 30)) return fail(SDV_ERR_SHAPE, "too many query rows");
  st = check_workspace(SDV_OP_VERIFY_SPARSE, workspace, workspace_bytes, rows_cap, num_q_heads,
                       kv->head_dim, num_splits);
  if (st) return st;
  if (B > 0 && (!block_table || !out || (!scores && !topk_idx)))
    return fail(SDV_ERR_NULL_POINTER, "block_table, %s and out must be non-null",
                scores ? "scores" : "topk_idx");
  if (reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "out must be 16-byte aligned");
  sdv::AttnArgs a{};
  a.q = q; a.q_dt = q_dt; a.qo_indptr = qo_indptr; a.kv_len = kv_len; a.B = B;
  a.max_qo_len = max_qo_len; a.num_q_heads = num_q_heads; a.num_kv_heads = kv->num_kv_heads;
  a.head_dim = kv->head_dim; a.kv_dt = kv->kv_dtype; a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale; a.softmax_scale = softmax_scale; a.num_splits = num_splits;
  a.out = out; a.out_dt = out_dt; a.dev_err = dev_err;
  const bool select_in_kernel = scores && fam != kFamilyValu && sdv::mfma_supported(a) &&
                                max_pages <= sdv::kFusedTopkMaxPages;
  if (scores && !select_in_kernel && B > 0 && !topk_out)
    return fail(SDV_ERR_NULL_POINTER, "topk_idx must hold the selection: the vector-ALU "
                "kernels, and tables over %d pages, select in a launch of its own",
                sdv::kFusedTopkMaxPages);
  if (scores && !select_in_kernel && max_pages > 4096)
    return fail(SDV_ERR_SHAPE, "max_pages %d > 4096 for the page selection", max_pages);
  if (B == 0) return ok();
  hipError_t e;
  if (scores && !select_in_kernel) {
    // the selection as its own launch, then the attention over it
    e = sdv::launch_topk(scores, qo_indptr, kv_len, B, max_qo_len, kv->num_kv_heads, max_pages,
                         top_k, topk_out, cnt_out, dev_err, stream);
    if (e != hipSuccess) return hip_status(e, name);
    topk_idx = topk_out;
  }
  split_workspace(workspace, rows_cap, num_q_heads, kv->head_dim, num_splits, &a.part_o, &a.part_lse);
  sdv::SparseSource src{kv->k, kv->v, kv->page_stride, kv->num_pages, block_table, bt_stride,
                        max_pages, select_in_kernel ? nullptr : topk_idx, top_k,
                        select_in_kernel ? scores : nullptr, topk_out, cnt_out};
  if (fam == kFamilyValu || !sdv::mfma_supported(a)) e = sdv::launch_attn_sparse_valu(a, src, stream);
  else if (fam == kFamilyRing) e = sdv::launch_attn_sparse_stream(a, src, stream);
  else e = sdv::launch_attn_sparse_waves(a, src, stream);
  if (e != hipSuccess) return hip_status(e, name);
  if (num_splits > 1) {
    e = sdv::launch_combine(a.part_o, a.part_lse, num_splits, static_cast<int32_t>(rows_cap),
                            qo_indptr, qo_indptr + B, num_q_heads, kv->head_dim, out, out_dt,
                            nullptr, stream);
    if (e != hipSuccess) return hip_status(e, name);
  }
  return ok();
}

extern "C" {

int32_t verify_attention_sparse(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                                const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                int32_t num_q_heads, const sdv_paged_kv* kv,
                                const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
                                const int32_t* topk_idx, int32_t top_k, float softmax_scale,
                                int32_t num_splits, void* workspace, size_t workspace_bytes,
                                void* out, int32_t out_dt, int32_t* dev_err,
                                hipStream_t stream) {
  return sparse_attention(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, kv, block_table,
                          max_pages, bt_stride, topk_idx, nullptr, nullptr, nullptr, top_k,
                          softmax_scale, num_splits, workspace, workspace_bytes, out, out_dt,
                          dev_err, stream, "verify_attention_sparse launch", kFamilyAuto);
}

int32_t verify_attention_sparse_select(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                                       const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                       int32_t num_q_heads, const sdv_paged_kv* kv,
                                       const int32_t* block_table, int32_t max_pages,
                                       int32_t bt_stride, const float* scores, int32_t top_k,
                                       int32_t* topk_idx, int32_t* topk_cnt,
                                       float softmax_scale, int32_t num_splits, void* workspace,
                                       size_t workspace_bytes, void* out, int32_t out_dt,
                                       int32_t* dev_err, hipStream_t stream) {
  if (B > 0 && !scores) return fail(SDV_ERR_NULL_POINTER, "scores must be non-null");
  return sparse_attention(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, kv, block_table,
                          max_pages, bt_stride, nullptr, scores, topk_idx, topk_cnt, top_k,
                          softmax_scale, num_splits, workspace, workspace_bytes, out, out_dt,
                          dev_err, stream, "verify_attention_sparse_select launch", kFamilyAuto);
}

int32_t lse_combine(const float* partial_out, const float* partial_lse, int32_t num_splits,
                    int32_t num_rows, int32_t num_heads, int32_t head_dim, void* out,
                    int32_t out_dt, float* lse_out, hipStream_t stream) {
  if (num_splits < 1 || num_rows < 0 || num_heads < 1)
    return fail(SDV_ERR_SHAPE, "num_splits %d, num_rows %d, num_heads %d", num_splits, num_rows,
                num_heads);
  if (!valid_head_dim(head_dim)) return fail(SDV_ERR_SHAPE, "head_dim %d", head_dim);
  if (!valid_out_dtype(out_dt)) return fail(SDV_ERR_DTYPE, "out dtype %d", out_dt);
  if (num_rows > 0 && (!partial_out || !partial_lse || !out))
    return fail(SDV_ERR_NULL_POINTER, "partial_out, partial_lse and out must be non-null");
  if (num_rows == 0) return ok();
  return hip_status(sdv::launch_combine(partial_out, partial_lse, num_splits, num_rows, nullptr,
                                        nullptr, num_heads, head_dim, out, out_dt, lse_out,
                                        stream),
                    "lse_combine launch");
}

int32_t sdv_fill_u32(void* dst, size_t bytes, uint32_t pattern, hipStream_t stream) {
  if (bytes == 0) return ok();
  if (!dst) return fail(SDV_ERR_NULL_POINTER, "dst must be non-null");
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "fill needs 16-byte aligned size and address");
  return hip_status(sdv::launch_fill_u32(dst, bytes, pattern, stream), "sdv_fill_u32 launch");
}

int32_t sdv_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                       hipStream_t stream) {
  if (bytes == 0) return ok();
  if (!src || !sink) return fail(SDV_ERR_NULL_POINTER, "src and sink must be non-null");
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "probe needs 16-byte aligned size and address");
  if (blocks < 1 || blocks > (1 << 20)) return fail(SDV_ERR_SHAPE, "blocks %d", blocks);
  return hip_status(sdv::launch_read_probe(src, bytes, sink, blocks, stream),
                    "sdv_read_probe launch");
}

int32_t sdv_read_units_probe(const void* base, size_t base_bytes, const int64_t* units,
                             int64_t n_units, int32_t unit_bytes, uint32_t* sink, int32_t blocks,
                             hipStream_t stream) {
  if (n_units == 0) return ok();
  if (!base || !units || !sink) return fail(SDV_ERR_NULL_POINTER, "base, units and sink must be non-null");
  if (unit_bytes != 4096 && unit_bytes != 8192 && unit_bytes != 16384)
    return fail(SDV_ERR_SHAPE, "unit_bytes %d (4096, 8192 or 16384)", unit_bytes);
  if (n_units < 0 || reinterpret_cast<uintptr_t>(base) % 16 != 0)
    return fail(SDV_ERR_SHAPE, "n_units %lld, base alignment", static_cast<long long>(n_units));
  if (blocks < 1 || blocks > (1 << 20)) return fail(SDV_ERR_SHAPE, "blocks %d", blocks);
  return hip_status(sdv::launch_read_units_probe(base, units, n_units,
                                                 static_cast<int64_t>(base_bytes / unit_bytes),
                                                 unit_bytes, sink, blocks, stream),
                    "sdv_read_units_probe launch");
}

}  // extern "C"

#ifdef SDV_XCHECK
// Cross-check build: the attention entry points with the kernel family as an argument of
// the call (declared in tests' ctypes binding only; the product library does not export
// them).  An unknown family is SDV_ERR_SHAPE; a family that does not serve the arguments
// falls back to the default kernel, as documented per family in the test binding.
extern "C" {

#define SDV_XCHECK_FAMILY()                                                            \
  if (!valid_family(family)) return fail(SDV_ERR_SHAPE, "kernel family %d", family);

int32_t sdv_xcheck_verify_attention_dense(
    int32_t family, const void* q, int32_t q_dt, const int32_t* qo_indptr,
    const int32_t* kv_len, int32_t B, int32_t max_qo_len, int32_t num_q_heads,
    const sdv_subpage_view* view, const int32_t* sub_offsets, int32_t max_sub_pages,
    float softmax_scale, int32_t num_splits, void* workspace, size_t workspace_bytes, void* out,
    int32_t out_dt, int32_t* dev_err, hipStream_t stream) {
  SDV_XCHECK_FAMILY()
  return dense_offsets_call(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, view,
                            sub_offsets, max_sub_pages, softmax_scale, num_splits, workspace,
                            workspace_bytes, out, out_dt, dev_err, stream, family);
}

int32_t sdv_xcheck_verify_attention_dense_view(
    int32_t family, const void* q, int32_t q_dt, const int32_t* qo_indptr,
    const int32_t* kv_len, int32_t B, int32_t max_qo_len, int32_t num_q_heads,
    const sdv_subpage_view* view, const int32_t* block_table, int32_t max_blocks,
    int32_t bt_stride, float softmax_scale, int32_t num_splits, void* workspace,
    size_t workspace_bytes, void* out, int32_t out_dt, int32_t* dev_err, hipStream_t stream) {
  SDV_XCHECK_FAMILY()
  return dense_view_call(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, view,
                         block_table, max_blocks, bt_stride, softmax_scale, num_splits,
                         workspace, workspace_bytes, out, out_dt, dev_err, stream, family);
}

int32_t sdv_xcheck_verify_attention_sparse(
    int32_t family, const void* q, int32_t q_dt, const int32_t* qo_indptr,
    const int32_t* kv_len, int32_t B, int32_t max_qo_len, int32_t num_q_heads,
    const sdv_paged_kv* kv, const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
    const int32_t* topk_idx, int32_t top_k, float softmax_scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes, void* out, int32_t out_dt, int32_t* dev_err,
    hipStream_t stream) {
  SDV_XCHECK_FAMILY()
  return sparse_attention(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, kv, block_table,
                          max_pages, bt_stride, topk_idx, nullptr, nullptr, nullptr, top_k,
                          softmax_scale, num_splits, workspace, workspace_bytes, out, out_dt,
                          dev_err, stream, "verify_attention_sparse launch", family);
}

int32_t sdv_xcheck_verify_attention_sparse_select(
    int32_t family, const void* q, int32_t q_dt, const int32_t* qo_indptr,
    const int32_t* kv_len, int32_t B, int32_t max_qo_len, int32_t num_q_heads,
    const sdv_paged_kv* kv, const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
    const float* scores, int32_t top_k, int32_t* topk_idx, int32_t* topk_cnt,
    float softmax_scale, int32_t num_splits, void* workspace, size_t workspace_bytes, void* out,
    int32_t out_dt, int32_t* dev_err, hipStream_t stream) {
  SDV_XCHECK_FAMILY()
  if (B > 0 && !scores) return fail(SDV_ERR_NULL_POINTER, "scores must be non-null");
  return sparse_attention(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, kv, block_table,
                          max_pages, bt_stride, nullptr, scores, topk_idx, topk_cnt, top_k,
                          softmax_scale, num_splits, workspace, workspace_bytes, out, out_dt,
                          dev_err, stream, "verify_attention_sparse_select launch", family);
}

int32_t sdv_xcheck_verify_attention_paged(
    int32_t family, const void* q, int32_t q_dt, const int32_t* qo_indptr,
    const int32_t* kv_len, int32_t B, int32_t max_qo_len, int32_t num_q_heads,
    const sdv_paged_kv* kv, const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
    float softmax_scale, int32_t num_splits, void* workspace, size_t workspace_bytes, void* out,
    int32_t out_dt, int32_t* dev_err, hipStream_t stream) {
  SDV_XCHECK_FAMILY()
  return paged_call(q, q_dt, qo_indptr, kv_len, B, max_qo_len, num_q_heads, kv, block_table,
                    max_pages, bt_stride, softmax_scale, num_splits, workspace, workspace_bytes,
                    out, out_dt, dev_err, stream, family);
}

#undef SDV_XCHECK_FAMILY

}  // extern "C"
#endif  // SDV_XCHECK
