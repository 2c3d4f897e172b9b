/*
 * sdv.h — C ABI of the MI355X (gfx950) speculative-decoding verify-attention library.
 *
 * The library computes the multi-token verify step of speculative decoding over a
 * paged KV cache.  Each request r contributes qo_len = 1 + draft_len query tokens;
 * token t (0 <= t < qo_len) attends the first
 *
 *     bound(r, t) = kv_len[r] - qo_len[r] + t + 1
 *
 * positions of its request, where kv_len counts the request's own verify tokens.
 * (Source: "[TRTLLM-14093][feat] Eagle3 for M3 MSA path + CUDA graphs
 * compatibility", MSA multi-token verify commit: the inclusive causal bound with
 * offset kv_len - qo_len gives this ladder.)
 *
 * Two variants:
 *   dense  — GQA draft-layer attention through a non-owning 32-token sub-page view
 *            of 128-token physical pages:  kv_subpage_view_init, then
 *            verify_attention_dense.
 *   sparse — block-sparse target layer:  proxy_page_scores -> ladder_topk_pages ->
 *            verify_attention_sparse.
 *
 * Conventions shared by every entry point
 *   - Return value: SDV_OK (0) or a nonzero sdv_status.  On failure nothing was
 *     enqueued and sdv_last_error() holds a message (thread-local).
 *   - All argument checks run on the host before any HIP call, so every rejection
 *     is reproducible without a GPU.
 *   - Pointers marked "device" are caller-owned device memory; the library never
 *     allocates, frees, synchronises or creates streams, and keeps no pointer after
 *     the call returns.  Every kernel goes onto `stream` (0 = the default stream),
 *     so the calls can be captured into a HIP graph.
 *   - Grids are sized from capacities (batch, max_qo_len, page-table width), never
 *     from current lengths: kv_len and qo_indptr are read on the device each launch,
 *     so a captured launch stays correct when the lengths change.
 *   - Query rows: request r owns rows qo_indptr[r] .. qo_indptr[r+1]-1 of q, out,
 *     scores and top-k arrays; row-indexed buffers are sized for B * max_qo_len rows.
 *   - Query head hq belongs to KV head hq / (num_q_heads / num_kv_heads).
 *   - dev_err (nullable, device int32): a kernel that meets inconsistent data ORs an
 *     SDV_DEVERR_* bit into it and skips the affected request or row; its outputs are
 *     then unspecified.  Clear it before the call if you want to read it after.
 */
#ifndef SDV_H
#define SDV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum sdv_status {
  SDV_OK = 0,
  SDV_ERR_NULL_POINTER = 1,   /* a required pointer is null                          */
  SDV_ERR_DTYPE = 2,          /* unsupported element type or type combination        */
  SDV_ERR_GEOMETRY = 3,       /* page geometry the native P128 draft view cannot serve */
  SDV_ERR_SHAPE = 4,          /* sizes out of the supported range                     */
  SDV_ERR_WORKSPACE = 5,      /* workspace missing or smaller than sdv_workspace_bytes */
  SDV_ERR_HIP = 6,            /* a HIP launch reported an error                        */
} sdv_status;

typedef enum sdv_dtype {
  SDV_F32 = 0,                /* IEEE binary32                                         */
  SDV_BF16 = 1,               /* bfloat16                                              */
  SDV_FP8_E4M3 = 2,           /* OCP E4M3FN (bias 7, max 448, no inf), with an fp32
                                 per-tensor scale: value = decode(byte) * scale        */
} sdv_dtype;

/* Device error bits. */
#define SDV_DEVERR_QO_LEN 1       /* qo_len < 1, qo_len > max_qo_len, kv_len < qo_len,
                                     or qo_indptr rows beyond B * max_qo_len           */
#define SDV_DEVERR_KV_CAPACITY 2  /* kv_len larger than the page table can address    */
#define SDV_DEVERR_PAGE_RANGE 4   /* a slot, page or sub-page index outside the pool   */
#define SDV_DEVERR_TOPK_INDEX 8   /* a top-k page index >= the token's valid pages     */
#define SDV_DEVERR_COPY_RANGE 16  /* a copy descriptor outside its buffers or not a
                                     multiple of 16 bytes                              */

#define SDV_PHYS_PAGE 128
#define SDV_SUB_PAGE 32

/* ---------------------------------------------------------------------------------
 * Dense draft layer: the non-owning P32 view of P128 pages.
 *
 * Pool geometry (sources: "[None][perf] wrap up eagle changes in m3 side branch",
 * commit fixing the draft view's index scale; "[None][perf] Default Minimax-m3 to
 * unified draft-target kv manager + change CI test to GQA eagle head", section Root
 * causes and fixes, item 2 "Grouped-HND draft KV transfer"):
 *   - the view is rooted at the draft layer's K page of slot 0 (k_root);
 *   - counted in 128-token pages from the root, slot s's K page is s * slot_stride
 *     and its V page s * slot_stride + 1 (kv_offset = 1); slot_stride is the view's
 *     index scale, and the pool's own page-index scale is NOT used (it may differ,
 *     e.g. 171 against a stride of 8);
 *   - each 128-token page is four independent head-major 32-token groups,
 *     logically [group = 4][num_kv_heads][32][head_dim], elements contiguous.
 *   So P32 page x (counted from k_root) holds element (head h, token o, channel c)
 *   at element offset ((x * num_kv_heads + h) * 32 + o) * head_dim + c.
 * ------------------------------------------------------------------------------- */
typedef struct sdv_subpage_geom {
  int32_t phys_page;        /* must be 128                                             */
  int32_t sub_page;         /* must be 32                                              */
  int32_t num_kv_heads;     /* >= 1                                                    */
  int32_t head_dim;         /* 64 or 128                                               */
  int32_t slot_stride;      /* P128 pages per slot, >= 2                               */
  int32_t kv_offset;        /* V page minus K page within a slot; must be 1            */
  int32_t num_layers;       /* layers the view spans; must be 1 (single-layer view)    */
  int32_t num_slots;        /* slots addressable from k_root; ids must be < num_slots  */
  int32_t pool_index_scale; /* the pool's page-index scale: recorded, never used       */
  int32_t kv_dtype;         /* sdv_dtype of the stored K/V                             */
  float k_scale;            /* dequantisation scales (1.0 unless fp8)                 */
  float v_scale;
  const void* k_root;       /* device: first element of slot 0's draft-layer K page    */
} sdv_subpage_geom;

/* Plain value describing a validated view; produced by kv_subpage_view_init. */
typedef struct sdv_subpage_view {
  const void* k_root;
  int32_t kv_dtype;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t index_scale;      /* = slot_stride                                           */
  int32_t num_slots;
  float k_scale;
  float v_scale;
  int64_t num_sub_pages;    /* P32 pages from k_root through the last slot's V page:
                               4 * ((num_slots - 1) * slot_stride + 2)                 */
} sdv_subpage_view;

/*
 * kv_subpage_view_init — validate the draft view's geometry and write, for every
 * request and every 32-token sub-page of its block-table capacity, the P32 page
 * indices of its K and V:
 *     slot = block_table[r * bt_stride + i / 4],  g = i % 4,
 *     sub_offsets[r][0][i] = 4 * slot_stride * slot + g,
 *     sub_offsets[r][1][i] = sub_offsets[r][0][i] + 4.
 * Padding entries are left as the caller wrote them (0 = slot 0, valid memory; the
 * pages keep the padding instead of clamping it: same PR #18066, commit removing
 * code made redundant by the native P128 draft view).
 *
 * geom        host, read during the call.
 * block_table device int32 [B][bt_stride], P128 slot ids; columns >= max_blocks unused.
 * sub_offsets device int32 out [B][2][4 * max_blocks].
 * view_out    host out: the validated view (plain value; copy freely).
 * dev_err     nullable; SDV_DEVERR_PAGE_RANGE for a slot id outside [0, num_slots)
 *             (that entry is then written as slot 0).
 * Errors: SDV_ERR_GEOMETRY ("native P128 draft view unavailable: <reason>") for a
 * page other than 128, sub-page other than 32, kv_offset != 1, num_layers != 1,
 * slot_stride < 2, head_dim not 64/128, or num_slots * slot_stride * 4 >= 2^31.
 */
int32_t kv_subpage_view_init(const sdv_subpage_geom* geom, const int32_t* block_table,
                             int32_t B, int32_t max_blocks, int32_t bt_stride,
                             int32_t* sub_offsets, sdv_subpage_view* view_out,
                             int32_t* dev_err, hipStream_t stream);

/*
 * verify_attention_dense — dense GQA verify attention through the P32 view.
 *   out[row(r,t)][hq] = sum_{j < bound(r,t)} softmax_j(scale * q . k_j) * v_j
 * over the request's logical positions j, K/V gathered through sub_offsets
 * (position j lives in P32 page sub_offsets[r][.][j / 32], token j % 32).
 * Float32 accumulation.  (Sources: PR #17835 Description — the Eagle3 drafter reads
 * its KV through the non-owning sub-page view; PR #3 MSA verify commit — the ladder.)
 *
 * q            device [B*max_qo_len rows capacity][num_q_heads][head_dim], q_dt;
 *              16-byte aligned (every call that takes q checks this).
 * qo_indptr    device int32 [B+1];  kv_len device int32 [B].
 * view         host: from kv_subpage_view_init.
 * sub_offsets  device int32 [B][2][max_sub_pages]; kv_len[r] <= 32 * max_sub_pages.
 * num_splits   >= 1: the most partial results per (request, KV head).  Each request's
 *              sub-pages are cut into contiguous runs, run s being split s; partials
 *              are merged by the log-sum-exp combine.  The default matrix-core kernel
 *              (B <= 512) cuts a pair of n sub-pages into k = ceil(n / C) near-equal
 *              runs, C the smallest length for which every pair's runs fit the
 *              workgroups the GPU holds at once, at least ceil(longest request's
 *              sub-pages / num_splits) (so k <= num_splits) and at most 1024, chosen on
 *              the device from kv_len; splits past a pair's k are empty.  The others
 *              take runs of one length C for the whole call: about the call's total
 *              sub-pages over all pairs divided by the workgroups the GPU holds at once,
 *              within the same bounds (the vector-ALU kernels: C = ceil(max_sub_pages /
 *              num_splits)).  With at
 *              least two (request, KV head) pairs per compute unit, num_splits >= 2,
 *              B <= 2048 and ceil(max_sub_pages / (num_splits - 1)) <= 1024, the call
 *              runs persistent instead: the pairs are laid end to end and every
 *              workgroup attends an equal range of sub-pages, num_splits bounding how
 *              many workgroups share one pair.
 *              Trailing splits of short requests are empty.  num_splits = 1 needs no
 *              workspace.  A split holds at most 1024 sub-pages, so
 *              ceil(max_sub_pages / num_splits) > 1024 is SDV_ERR_SHAPE.
 * workspace    device, >= sdv_workspace_bytes(SDV_OP_VERIFY_DENSE, B*max_qo_len,
 *              num_q_heads, head_dim, num_splits) bytes (nullable when that is 0).
 * out          device [rows][num_q_heads][head_dim], out_dt (F32 or BF16); 16-byte
 *              aligned.
 * Supported: q_dt F32 with F32 K/V; q_dt BF16 with BF16 or FP8 K/V; head_dim 64 or
 * 128; num_q_heads % num_kv_heads == 0; max_qo_len * G <= 64.
 */
int32_t verify_attention_dense(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                               const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                               int32_t num_q_heads, const sdv_subpage_view* view,
                               const int32_t* sub_offsets, int32_t max_sub_pages,
                               float softmax_scale, int32_t num_splits, void* workspace,
                               size_t workspace_bytes, void* out, int32_t out_dt,
                               int32_t* dev_err, hipStream_t stream);

/*
 * verify_attention_dense_view — kv_subpage_view_init's page indices and
 * verify_attention_dense in one launch: the attention kernels compute each 32-token
 * sub-page's P32 K and V indices from the block table as the view defines them
 * (slot = block_table[r * bt_stride + i / 4], K = 4 * index_scale * slot + i % 4,
 * V = K + 4), so no sub_offsets array is written or read.  (Sources: PR #17835
 * Description and item 2 — the non-owning P32 view of the P128 pages; PR #18066
 * draft-view index-scale commit.)
 *
 * view         host: a view validated by kv_subpage_view_init (a call with B = 0 only
 *              validates the geometry and fills the view, launching nothing).
 * block_table  device int32 [B][bt_stride] P128 slot ids; columns >= max_blocks unused;
 *              kv_len[r] <= 128 * max_blocks.
 * A slot id outside [0, num_slots) sets SDV_DEVERR_PAGE_RANGE in dev_err and its
 * sub-pages are left out (the two-call path reads slot 0 there; both outputs are then
 * unspecified for that request).  Other arguments, limits and results as in
 * verify_attention_dense with max_sub_pages = 4 * max_blocks.
 */
int32_t verify_attention_dense_view(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                                    const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                    int32_t num_q_heads, const sdv_subpage_view* view,
                                    const int32_t* block_table, int32_t max_blocks,
                                    int32_t bt_stride, float softmax_scale, int32_t num_splits,
                                    void* workspace, size_t workspace_bytes, void* out,
                                    int32_t out_dt, int32_t* dev_err, hipStream_t stream);

/*
 * verify_attention_dense_view_noalloc — verify_attention_dense_view for callers that
 * cannot allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Arguments, results and errors
 * as verify_attention_dense_view without workspace / workspace_bytes: the split-KV
 * partials (sdv_workspace_bytes(SDV_OP_VERIFY_DENSE, B * max_qo_len, num_q_heads,
 * head_dim, num_splits) bytes) go to a device scratch array of
 * SDV_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the
 * process ends.  A call that needs more is SDV_ERR_WORKSPACE (use fewer splits or rows,
 * or the workspace entry point).  The call allocates nothing; the first call on a device
 * looks up that device's scratch address.  Every call on one GPU shares that GPU's
 * scratch, so calls that overlap in time on one GPU (concurrent streams, or host threads
 * enqueueing on different streams) race and give unspecified results; calls ordered on
 * one stream do not.  Nothing in the scratch needs to start at zero.
 */
#define SDV_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int32_t verify_attention_dense_view_noalloc(const void* q, int32_t q_dt,
                                            const int32_t* qo_indptr, const int32_t* kv_len,
                                            int32_t B, int32_t max_qo_len, int32_t num_q_heads,
                                            const sdv_subpage_view* view,
                                            const int32_t* block_table, int32_t max_blocks,
                                            int32_t bt_stride, float softmax_scale,
                                            int32_t num_splits, void* out, int32_t out_dt,
                                            int32_t* dev_err, hipStream_t stream);

/* ---------------------------------------------------------------------------------
 * Sparse target layer over ordinary head-major 128-token pages: page p of K holds
 * [num_kv_heads][128][head_dim] contiguous elements at k + p * page_stride (V alike).
 * Request r's position j is token j % 128 of page block_table[r * bt_stride + j/128].
 * ------------------------------------------------------------------------------- */
typedef struct sdv_paged_kv {
  const void* k;            /* device: page 0 of K                                     */
  const void* v;            /* device: page 0 of V                                     */
  int64_t page_stride;      /* elements between pages, >= num_kv_heads * 128 * head_dim */
  int32_t num_pages;        /* page ids must lie in [0, num_pages)                     */
  int32_t page_size;        /* must be 128                                             */
  int32_t num_kv_heads;
  int32_t head_dim;         /* 64 or 128                                               */
  int32_t kv_dtype;         /* sdv_dtype                                               */
  float k_scale;
  float v_scale;
} sdv_paged_kv;

/*
 * proxy_page_scores — score every page of every request for every verify token in
 * one pass over K (PR #3 MSA verify commit: the proxy "OnlyScore" pass is natively
 * multi-token under the ladder bound; its formula is not on the pages and is fixed
 * here as):
 *   scores[row(r,t)][h][p] = max_{hq in group h} q[row][hq] . ksum(r,t,h,p),
 *   ksum = sum of K[j][h][:] over positions j of page p with j < bound(r,t),
 * and -inf for pages with no such position.  Unscaled (no softmax or fp8 scale).
 * Evaluated in float32 in a fixed order: ksum accumulated one position at a time in
 * ascending order starting from 0; products q[c] * ksum[c] rounded separately (no
 * fused multiply-add); summed by recursive halving over channels (c with c + n/2,
 * n = head_dim, head_dim/2, ..., 2); -0 returned as +0.
 *
 * scores  device float [B*max_qo_len][num_kv_heads][max_pages]; entries for pages
 *         p < ceil(kv_len[r] / 128) of each request are written, others untouched.
 * block_table device int32 [B][bt_stride], request-local page p -> physical page.
 * Supported: q F32 or BF16; K F32, BF16 or FP8; head_dim 64 or 128;
 * max_qo_len * G * head_dim <= 8192; B <= 65535; max_pages <= 131070.
 */
int32_t proxy_page_scores(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                          const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                          int32_t num_q_heads, const sdv_paged_kv* kv,
                          const int32_t* block_table, int32_t max_pages, int32_t bt_stride,
                          float* scores, int32_t* dev_err, hipStream_t stream);

/*
 * ladder_topk_pages — per (token, KV head): the k_eff = min(top_k, n_valid) best
 * pages among p < n_valid(r,t) = ceil(bound(r,t) / 128), ordered by score
 * descending then page index ascending (ties go to the lower page), written in rank
 * order and padded with -1 (PR #3 MSA verify commit: per-token ladder valid-page
 * counts, so a draft token cannot select pages past its own bound).
 *
 * scores    device float [B*max_qo_len][num_kv_heads][max_pages] (reads p < n_valid).
 * topk_idx  device int32 out [B*max_qo_len][num_kv_heads][top_k].
 * topk_cnt  device int32 out [B*max_qo_len][num_kv_heads], nullable.
 * Supported: page_size 128; 1 <= top_k <= 1024; max_pages <= 4096; B <= 65535.
 */
int32_t ladder_topk_pages(const float* scores, const int32_t* qo_indptr,
                          const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                          int32_t num_kv_heads, int32_t max_pages, int32_t page_size,
                          int32_t top_k, int32_t* topk_idx, int32_t* topk_cnt,
                          int32_t* dev_err, hipStream_t stream);

/*
 * verify_attention_sparse — sparse GQA verify attention: token t, query head hq of
 * KV head h attends position j iff page j / 128 is in topk_idx[row(r,t)][h][:] and
 * j < bound(r,t).  Each (request, KV head) reads every page selected by any of its
 * tokens once (the union), not once per token.  num_splits splits that union into
 * near-equal contiguous chunks (split-KV with a log-sum-exp combine).
 *
 * topk_idx device int32 [B*max_qo_len][num_kv_heads][top_k], -1 = unused slot.
 * Other arguments as in proxy_page_scores and verify_attention_dense.
 * Supported: as verify_attention_dense; max_pages <= 16384.
 */
int32_t verify_attention_sparse(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                                const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                int32_t num_q_heads, const sdv_paged_kv* kv,
                                const int32_t* block_table, int32_t max_pages,
                                int32_t bt_stride, const int32_t* topk_idx, int32_t top_k,
                                float softmax_scale, int32_t num_splits, void* workspace,
                                size_t workspace_bytes, void* out, int32_t out_dt,
                                int32_t* dev_err, hipStream_t stream);

/*
 * verify_attention_sparse_select — ladder_topk_pages and verify_attention_sparse in one
 * launch: each attention workgroup selects its (request, KV head)'s pages from scores
 * itself (one wave per verify token, the same selection as ladder_topk_pages: score
 * descending, page ascending on ties, among each token's own n_valid pages) and attends
 * them.  (Sources: PR #3 MSA verify commit — per-token ladder top-k; the proxy pass and
 * the selection feed the sparse attention of the same step.)
 *
 * scores    device float [B*max_qo_len][num_kv_heads][max_pages] (proxy_page_scores).
 * topk_idx  device int32 [B*max_qo_len][num_kv_heads][top_k] OUT, nullable: the
 *           selection as ladder_topk_pages writes it.  Required (SDV_ERR_NULL_POINTER
 *           otherwise) when the selection runs as a launch of its own first: kernel
 *           families 1 and 2, f32 query/KV, and max_pages > 1024 (the in-kernel
 *           selection holds up to 1024 pages).  Rows of requests flagged on the device
 *           are not written.
 * topk_cnt  device int32 [B*max_qo_len][num_kv_heads] OUT, nullable.
 * Other arguments as in verify_attention_sparse; max_pages <= 4096.
 */
int32_t verify_attention_sparse_select(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                                       const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                                       int32_t num_q_heads, const sdv_paged_kv* kv,
                                       const int32_t* block_table, int32_t max_pages,
                                       int32_t bt_stride, const float* scores, int32_t top_k,
                                       int32_t* topk_idx, int32_t* topk_cnt,
                                       float softmax_scale, int32_t num_splits, void* workspace,
                                       size_t workspace_bytes, void* out, int32_t out_dt,
                                       int32_t* dev_err, hipStream_t stream);

/*
 * verify_attention_paged — dense GQA verify attention over ordinary head-major P128
 * pages, for the target model's dense layers: token t, query head hq of KV head h
 * attends every position j < bound(r,t) of its request (the ladder mask; at qo_len = 1
 * it is ordinary decode attention).  Position j lives at token j % 128 of page
 * block_table[r][j / 128].  (Source: PR #3 MSA verify commit — the dense layers 0-2
 * take a ladder attention mask.)
 *
 * Arguments as in verify_attention_sparse, without topk_idx.  num_splits >= 1 as in
 * verify_attention_dense with the capacity 4 * max_pages 32-token blocks; each split
 * holds at most 1024 blocks, so ceil(4 * max_pages / num_splits) <= 1024.  With
 * num_splits >= 2, B <= 2048 and ceil(4 * max_pages / (num_splits - 1)) <= 1024 the
 * call runs persistent: the (request, KV head) pairs are laid end to end and every
 * workgroup attends an equal range of 32-token blocks, so num_splits bounds how many
 * workgroups share one pair rather than fixing where a pair is cut.
 * Supported: q BF16 with BF16 or FP8 K/V; head_dim 64 or 128; G * max_qo_len <= 64.
 * Errors as verify_attention_sparse; SDV_ERR_DTYPE for F32 q.
 */
int32_t verify_attention_paged(const void* q, int32_t q_dt, const int32_t* qo_indptr,
                               const int32_t* kv_len, int32_t B, int32_t max_qo_len,
                               int32_t num_q_heads, const sdv_paged_kv* kv,
                               const int32_t* block_table, int32_t max_pages,
                               int32_t bt_stride, float softmax_scale, int32_t num_splits,
                               void* workspace, size_t workspace_bytes, void* out,
                               int32_t out_dt, int32_t* dev_err, hipStream_t stream);

/*
 * stage_verify_kv_paged — ladder KV slot staging into ordinary head-major P128 pages:
 * the K/V rows of the qo_len new tokens of every request are written at logical
 * positions kv_len - qo_len + t (kv_len counts them), i.e. token (j % 128) of page
 * block_table[r][j / 128] for j = kv_len - qo_len + t, across page boundaries.  Each
 * request addresses only its own block-table row with its own lengths, so after a
 * correction that shortens a request the next call writes at the corrected positions
 * and no other request's pages move.  (Source: PR #3 MSA verify commit — KV slot
 * staging generalises to the causal ladder; the overlap-correction fix.)
 *
 * k_new, v_new device [B*max_qo_len rows capacity][num_kv_heads][head_dim], rows in
 *              qo_indptr order, stored in the cache's dtype (new_dt must equal
 *              kv->kv_dtype: the bytes are copied, not converted); 16-byte aligned.
 * kv           host descriptor of the cache; the K/V storage kv->k / kv->v points
 *              to is WRITTEN (device memory the caller owns).
 * block_table  device int32 [B][bt_stride]; kv_len[r] <= 128 * max_pages.
 * dev_err      nullable; SDV_DEVERR_QO_LEN / _KV_CAPACITY / _PAGE_RANGE skip the
 *              affected request or row.
 * Rows of different requests must not share a (page, slot): the writes would race.
 */
int32_t stage_verify_kv_paged(const void* k_new, const void* v_new, int32_t new_dt,
                              const int32_t* qo_indptr, const int32_t* kv_len, int32_t B,
                              int32_t max_qo_len, const sdv_paged_kv* kv,
                              const int32_t* block_table, int32_t max_pages,
                              int32_t bt_stride, int32_t* dev_err, hipStream_t stream);

/*
 * stage_verify_kv_view — the same staging into the draft layer through the P32 view:
 * position j of request r goes to token j % 32 of P32 page sub_offsets[r][0][j / 32]
 * (K) and sub_offsets[r][1][j / 32] (V), element ((x * Hkv + h) * 32 + j % 32) * d
 * from the view root.  (Sources: PR #3 MSA verify commit, staging; PR #17835 item 2,
 * the grouped-HND layout of the view.)
 *
 * view, sub_offsets, max_sub_pages as for verify_attention_dense; the view's storage
 * is WRITTEN.  Other arguments as stage_verify_kv_paged; kv_len[r] <= 32 * max_sub_pages.
 */
int32_t stage_verify_kv_view(const void* k_new, const void* v_new, int32_t new_dt,
                             const int32_t* qo_indptr, const int32_t* kv_len, int32_t B,
                             int32_t max_qo_len, const sdv_subpage_view* view,
                             const int32_t* sub_offsets, int32_t max_sub_pages,
                             int32_t* dev_err, hipStream_t stream);

/*
 * greedy_accept — greedy acceptance of the draft tokens after the verify step.  Row t
 * of request r holds its t-th verify input token (row 0 the last accepted token, rows
 * 1 .. qo_len - 1 the drafts) and the target's logits after it.  The target's greedy
 * token after a row is the argmax of its logits (ties to the lowest index, NaN never
 * chosen, -1 for an all-NaN row).  Draft t + 1 is accepted while it equals the target
 * after row t for every earlier row; with a accepted drafts the step emits them and
 * the bonus token (the target after row a): a + 1 tokens, the acceptance length.  The
 * cache keeps the verify tokens through draft a, so the corrected kv_len is
 * kv_len - qo_len + 1 + a.  (Sources: PR #17835, Acceptance and accuracy evidence —
 * acceptance under greedy decoding, rate and mean length; PR #3 MSA verify commit —
 * the verify batch of qo_len = 1 + draft_len tokens.)
 *
 * logits       device [rows][vocab] (rows = qo_indptr[B] <= B*max_qo_len), F32 or BF16,
 *              16-byte aligned; vocab a multiple of 4 (F32) or 8 (BF16).
 * tokens       device int32 [rows]: the verify input tokens.
 * workspace    device, >= sdv_greedy_accept_workspace_bytes(B, max_qo_len, vocab,
 *              logits_dt) bytes, 8-byte aligned: each row's logits are reduced in
 *              parts of 4096 (F32) or 8192 (BF16) values whose maxima and indices (one
 *              64-bit key per part) it holds between the two launches.  Owned by the caller; contents on entry
 *              ignored; calls that share it on different streams race.
 * targets_out  device int32 [B*max_qo_len]: argmax per row, for the rows of every
 *              request whose rows lie inside [0, qo_indptr[B]) (rows past qo_indptr[B]
 *              untouched).
 * accept_out   device int32 [B]: accepted drafts a (-1 for a request with unusable
 *              lengths, flagged SDV_DEVERR_QO_LEN; rows reaching past qo_indptr[B] are
 *              unusable too).
 * emitted_out  device int32 [B][max_qo_len]: the a + 1 emitted tokens, -1 padded.
 * new_kv_len_out device int32 [B]: kv_len - qo_len + 1 + a (kv_len when flagged).
 * Errors: SDV_ERR_DTYPE (logits not F32/BF16), SDV_ERR_SHAPE (vocab, B, max_qo_len,
 * alignment, or B*max_qo_len*parts beyond 2^31 - 1 workgroups), SDV_ERR_NULL_POINTER,
 * SDV_ERR_WORKSPACE (workspace smaller than the size above).
 */
int32_t greedy_accept(const void* logits, int32_t logits_dt, int32_t vocab,
                      const int32_t* tokens, const int32_t* qo_indptr, const int32_t* kv_len,
                      int32_t B, int32_t max_qo_len, void* workspace, size_t workspace_bytes,
                      int32_t* targets_out, int32_t* accept_out, int32_t* emitted_out,
                      int32_t* new_kv_len_out, int32_t* dev_err, hipStream_t stream);

/* Workspace bytes greedy_accept needs: B * max_qo_len * ceil(vocab / (1024 * values per
 * 16 bytes)) * 8 (host only; 0 for arguments greedy_accept rejects). */
size_t sdv_greedy_accept_workspace_bytes(int32_t B, int32_t max_qo_len, int32_t vocab,
                                         int32_t logits_dt);

/* One byte-range copy: dst_base[dst_offset ..) = src_base[src_offset ..), `bytes` long. */
typedef struct sdv_copy_desc {
  int64_t src_offset;
  int64_t dst_offset;
  int64_t bytes;
} sdv_copy_desc;

/*
 * hnd_head_slice_descriptors — the head-slice transfer mapper for head-major pages
 * whose tokens may be split into token groups (host only, no HIP call).  A page of G
 * token groups is laid out [G][heads][page_tokens / G][head_dim]; the P32 view of the
 * draft layer's P128 pages is G = 4 ([4][local_head][32][d]), ordinary head-major
 * pages are G = 1.  For every listed page pair i and every group g it emits one
 * descriptor that moves heads [src_head_begin, + num_heads) of source page i to heads
 * [dst_head_begin, + num_heads) of destination page i — one descriptor per (layer,
 * K/V, token group) when the list enumerates the layers' K and V pages.  Mapping a
 * grouped page with G = 1 (one contiguous head slice per page) selects the right heads
 * only in the first group.  (Source: PR #17835, Root causes and fixes, item 2
 * "Grouped-HND draft KV transfer": the hnd_token_groups page-table field, default 1,
 * four groups for the shared draft K/V.)
 *
 * src_page_offsets, dst_page_offsets  host int64 [num_pages]: byte offset of each page
 *              from the source / destination base.
 * out          host [capacity]; descriptors in page-major, group-minor order.
 * count_out    host: num_pages * token_groups.
 * Errors: SDV_ERR_SHAPE for page_tokens not a multiple of token_groups, head ranges
 * outside [0, src_heads) / [0, dst_heads), or capacity < num_pages * token_groups.
 */
int32_t hnd_head_slice_descriptors(int32_t token_groups, int32_t src_heads,
                                   int32_t src_head_begin, int32_t dst_heads,
                                   int32_t dst_head_begin, int32_t num_heads,
                                   int32_t head_dim, int32_t kv_dtype, int32_t page_tokens,
                                   const int64_t* src_page_offsets,
                                   const int64_t* dst_page_offsets, int32_t num_pages,
                                   sdv_copy_desc* out, int32_t capacity, int32_t* count_out);

/*
 * copy_descriptors — execute byte-range copies on the device (the transfer engine's
 * work on one GPU; across GPUs the same descriptors drive peer copies).
 * descs device [num_descs]; every range must lie inside [0, src_bytes) / [0, dst_bytes)
 * and offsets and lengths must be multiples of 16 bytes, else that descriptor is
 * skipped and SDV_DEVERR_COPY_RANGE is flagged.  Destination ranges must not overlap
 * each other or the source.
 */
int32_t copy_descriptors(const void* src_base, size_t src_bytes, void* dst_base,
                         size_t dst_bytes, const sdv_copy_desc* descs, int32_t num_descs,
                         int32_t* dev_err, hipStream_t stream);

/*
 * lse_combine — merge split-KV partials:  LSE = log sum_s exp(lse[s]),
 * out = sum_s exp(lse[s] - LSE) * partial_out[s]; partials with lse = -inf are
 * skipped; a row with no live partial gets 0.
 * partial_out device float [num_splits][num_rows][num_heads][head_dim];
 * partial_lse device float [num_splits][num_rows][num_heads] (natural log);
 * out device [num_rows][num_heads][head_dim], out_dt F32 or BF16;
 * lse_out device float [num_rows][num_heads], nullable.
 */
int32_t lse_combine(const float* partial_out, const float* partial_lse, int32_t num_splits,
                    int32_t num_rows, int32_t num_heads, int32_t head_dim, void* out,
                    int32_t out_dt, float* lse_out, hipStream_t stream);

/* Operations that take a split-KV workspace (sdv_workspace_bytes' op argument). */
typedef enum sdv_op {
  SDV_OP_VERIFY_DENSE = 1,    /* verify_attention_dense, verify_attention_dense_view   */
  SDV_OP_VERIFY_SPARSE = 2,   /* verify_attention_sparse, verify_attention_sparse_select */
  SDV_OP_VERIFY_PAGED = 3,    /* verify_attention_paged                                 */
} sdv_op;

/* Workspace (bytes) the attention call `op` needs for q_rows_cap = B * max_qo_len query
 * rows and num_splits splits: the fp32 partial outputs [num_splits][q_rows_cap]
 * [num_q_heads][head_dim] and their log-sum-exps [num_splits][q_rows_cap][num_q_heads],
 * each padded to 256 bytes.  0 when num_splits == 1, for non-positive sizes, and for an
 * op not listed in sdv_op (the call itself then rejects a missing workspace). */
size_t sdv_workspace_bytes(int32_t op, int32_t q_rows_cap, int32_t num_q_heads,
                           int32_t head_dim, int32_t num_splits);

/* Static text for a status code. */
const char* sdv_status_string(int32_t status);

/* Message of the calling thread's most recent failed call ("" if none). */
const char* sdv_last_error(void);

/* Measurement helper: fill `bytes` (multiple of 16) of device memory with a 32-bit
 * pattern — used to evict caches between timed runs. */
int32_t sdv_fill_u32(void* dst, size_t bytes, uint32_t pattern, hipStream_t stream);

/* Measurement helper: read `bytes` (multiple of 16) of device memory once with 16-byte
 * loads using `blocks` workgroups of 256 threads; sink (device, >= blocks words) gets
 * an XOR fold so the reads are kept.  Its rate is the attainable streaming-read
 * bandwidth that the HBM-bound kernels are compared with. */
int32_t sdv_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                       hipStream_t stream);

/* Measurement helper: read a list of equal units once — unit u is the unit_bytes (4096,
 * 8192 or 16384) bytes at base + u * unit_bytes; units (device int64 [n_units]) outside
 * the base_bytes of memory at base are skipped — with `blocks` workgroups of 256
 * threads, four units in flight per workgroup; sink (device, >= blocks words) gets an
 * XOR fold.  Given a kernel's own gather list (say the K and V runs of every block a
 * dense call reads), its rate is the attainable bandwidth of that access pattern. */
int32_t sdv_read_units_probe(const void* base, size_t base_bytes, const int64_t* units,
                             int64_t n_units, int32_t unit_bytes, uint32_t* sink, int32_t blocks,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SDV_H */
