/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged-KV attention library.
 *
 * What it computes (vLLM API documentation pages):
 *   - vllm.v1.attention.backends.flashinfer_ts: attention of a uniform query
 *     block (query_len >= 1 tokens per request, grouped-query heads) over a
 *     paged cache [pages, Hkv, page_size, 2*D] whose K and V are the two
 *     halves of each page row (module docstring "Layout", _kv_views): the
 *     dense block with an optional sliding window applied as a page-aligned
 *     suffix (module docstring "Sliding window", _restrict_to_window), or the
 *     causal block with an exact per-token window (_get_plan: mask_type
 *     "causal", window_left = window - 1); the fp8 scale folding of
 *     FlashInferTSImpl.forward (bmm1_scale = scale * q_scale * k_scale,
 *     bmm2_scale = v_scale); and the cache write that precedes the step
 *     (do_kv_cache_update).
 *   - vllm.v1.attention.backends.fa_utils: Split-KV (num_splits) with a
 *     natural-log LSE returned per row and head (return_softmax_lse).
 *   - vllm.v1.attention.ops.dash_attention, flash_dash_attention: attention
 *     of one query over gathered segments, then the softmax over
 *     segment LSE + bias with empty segments masked out.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is DEVICE memory owned by the caller; the
 *     library never allocates, frees, synchronizes the host or reads device
 *     data on the host, so each call may be captured into a hipGraph.
 *   - Work is enqueued asynchronously on `stream` (NULL = null stream).
 *   - Return value: PA_OK or a negative pa_status.  pa_last_error() gives a
 *     thread-local message for the last failing call on this thread.
 *     Argument errors are detected before anything is enqueued.
 *   - LSE values are natural logarithms, fp32, one per (row, head) in
 *     [rows, heads] order.  A row that sees no key gets O = 0, LSE = -inf.
 *   - Query head h reads kv head h / (Hq / Hkv).
 *   - Element strides are counted in elements of the KV dtype.
 */
#ifndef PAGED_ATTN_H_
#define PAGED_ATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  PA_FP8_E4M3 is the OCP e4m3fn byte format: the pages keep an
 * fp8 cache in one-byte storage and hand its bytes to the kernel as e4m3
 * values (flashinfer_ts page, _kv_kernel_dtype). */
enum pa_dtype { PA_BF16 = 1, PA_FP16 = 2, PA_FP8_E4M3 = 3, PA_F32 = 4 };

enum pa_status {
  PA_OK = 0,
  PA_EINVAL = -1,     /* malformed argument (shape, stride, pointer, alignment) */
  PA_ENOTSUP = -2,    /* well-formed but unsupported (dtype or dtype combination) */
  PA_EWORKSPACE = -3, /* workspace missing or smaller than *_workspace_size() */
  PA_EHIP = -4        /* a kernel launch failed; see pa_last_error() */
};

/* A paged K/V cache.  Element (page, kv_head, slot, d) of K is at
 *   k + page*page_stride + kv_head*head_stride + slot*token_stride + d
 * and likewise for V from v.  head_dim must be contiguous (flashinfer_ts
 * module docstring: the only layout requirement).  For vLLM's
 * [pages, Hkv, P, 2*D] page, v = k + D and the strides are
 * (Hkv*P*2D, P*2D, 2D).  k, v must be 16-byte aligned and every stride a
 * multiple of 16 bytes, one token step (token_stride elements) at most 64 MiB
 * (PA_EINVAL otherwise).
 * Page indices read from the block table are clamped
 * to [0, num_pages) so a corrupt table cannot address outside the pool. */
typedef struct pa_kv_desc {
  const void* k;
  const void* v;
  int64_t page_stride;
  int64_t head_stride;
  int64_t token_stride;
  int32_t page_size;    /* tokens per page, >= 1 */
  int32_t num_kv_heads; /* Hkv */
  int32_t num_pages;    /* pages in the pool (bound for page indices) */
  int32_t dtype;        /* PA_BF16 | PA_FP16 | PA_FP8_E4M3 */
  float k_scale;        /* real K = k_scale * stored K (1 unless fp8) */
  float v_scale;        /* real V = v_scale * stored V (1 unless fp8) */
} pa_kv_desc;

/* Paged attention of a uniform query block: work partition, window restriction,
 * block-table gather, attention, and the split combine when splits > 1.
 *
 * q           [B, query_len, Hq, D] contiguous, q_dtype PA_BF16 | PA_FP16 |
 *             PA_FP8_E4M3.  A 16-bit cache must have the query's dtype; an
 *             fp8 cache takes either a 16-bit query (K and V are decoded
 *             exactly to that type) or an fp8 query (flashinfer_ts keeps q and K/V
 *             dtypes matched; the query arrives quantized): q.k then runs on
 *             fp8 MFMA and P.V in bf16.  An fp8 query's own scale is folded
 *             into `scale` by the caller (the page's bmm1_scale = scale *
 *             q_scale * k_scale).
 * block_table [B, bt_width] int32 with row stride bt_row_stride (elements);
 *             column j of row b names the pool page holding tokens
 *             [j*P, (j+1)*P) of request b.  Columns >= ceil(L_b / P) are
 *             never read.
 * seq_lens    [B] int32; L_b counts every key token including the query
 *             block itself (the block ends the sequence).  Values are
 *             clamped to [0, bt_width * page_size].
 * scale       softmax scale (the caller's 1/sqrt(D) or model value); the
 *             logit is scale * k_scale * q.k.
 * window      <= 0: no window.  > 0: request b sees only the keys from page
 *             floor((L_b - window - query_len + 1) / P) (clamped at 0) to
 *             L_b, i.e. the window suffix rounded down to a page
 *             (flashinfer_ts, _restrict_to_window).  Every query token of
 *             the block sees the same keys (dense mask).
 * num_splits  Split-KV policy.  1: one pass, no partials.  S > 1: the
 *             visible pages of each request are cut into S chunks of
 *             ceil(pages / S) pages, attended separately into the workspace
 *             and merged by the LSE-weighted combine.  0: chosen by the
 *             library from the static shape.  -c (c > 0): chunks of c pages,
 *             S = ceil(max visible pages / c).
 * out         [B, query_len, Hq, D], out_dtype PA_BF16 | PA_FP16 | PA_F32.
 * lse         [B, query_len, Hq] fp32 natural-log LSE, or NULL.
 * workspace   device scratch of >= paged_attn_workspace_size(...) bytes when
 *             the resolved split count exceeds 1 (else may be NULL): the
 *             fp32 partial outputs and LSEs of the splits, written by the
 *             attention kernel and read by the combine kernel that follows it
 *             on `stream`.  Its contents need no initialization; calls that
 *             share a workspace must not overlap in time.
 * B == 0 or query_len == 0 is a no-op returning PA_OK.  B * query_len and
 * (Hq / Hkv) * query_len must stay below 2^31 (PA_EINVAL otherwise).
 */
int paged_attn_run(const void* q, int32_t q_dtype, const pa_kv_desc* kv,
                   const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                   const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq, int32_t D,
                   float scale, int32_t window, int32_t num_splits,
                   void* out, int32_t out_dtype, float* lse,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of the device scratch paged_attn_run_noalloc keeps per GPU (96 MiB:
 * the Split-KV partials of a 32 x 16-token block of 32 heads at D = 128 in
 * 8 splits take 64.5 MiB). */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

/* paged_attn_run without a workspace argument, for callers that cannot
 * allocate device memory (code under hipGraph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, plan, kernels and results
 * as paged_attn_run; the Split-KV partials go to a static device array of
 * PA_NOALLOC_SCRATCH_BYTES that each GPU holds until the process ends.  The
 * call allocates and frees nothing.  Its first call on a device looks the
 * array's address up (hipGetSymbolAddress) for the device `stream` belongs
 * to.  A shape whose partials exceed the array (paged_attn_workspace_size >
 * PA_NOALLOC_SCRATCH_BYTES) returns PA_EWORKSPACE before anything is
 * enqueued.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race and give
 * wrong results.  Nothing in the array needs clearing between calls. */
int paged_attn_run_noalloc(const void* q, int32_t q_dtype, const pa_kv_desc* kv,
                           const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                           const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq,
                           int32_t D, float scale, int32_t window, int32_t num_splits,
                           void* out, int32_t out_dtype, float* lse, hipStream_t stream);

/* Causal query block (flashinfer_ts _get_plan: mask_type "causal" with
 * window_left = window - 1).  Arguments, plan, splits and workspace as
 * paged_attn_run; only the mask differs.  Token t of request b sits at
 * position L_b - query_len + t and sees the keys j <= that position; with
 * window > 0 also j >= position - (window - 1), an exact window of `window`
 * keys per token (no page rounding: pages before the first key any token of
 * the block can see are skipped, which changes no result).  A token with no
 * visible key (L_b < query_len) gets out = 0 and LSE = -inf. */
int paged_attn_run_causal(const void* q, int32_t q_dtype, const pa_kv_desc* kv,
                          const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                          const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq,
                          int32_t D, float scale, int32_t window, int32_t num_splits,
                          void* out, int32_t out_dtype, float* lse,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The split count paged_attn_run resolves num_splits to for this shape (>= 1).
 * The fa_utils page exposes num_splits as the Split-KV knob and leaves the
 * choice of splits to the kernel; the rule applied here for 0 (automatic) and
 * -c (chunks of c pages) is this library's own, and depends on the visible
 * page count, hence on Hkv, page_size, bt_width and window as well as on the
 * query shape.  Host only; a malformed shape gives 1. */
int32_t paged_attn_resolve_splits(int32_t B, int32_t query_len, int32_t Hq, int32_t Hkv,
                                  int32_t D, int32_t page_size, int32_t bt_width,
                                  int32_t window, int32_t num_splits);

/* The launch plan paged_attn_run uses for this shape (the Split-KV partition of
 * the fa_utils page, num_splits, and the work decomposition around it),
 * written to plan[0..5]:
 * split count S, pages per split (0 = ceil(visible pages / S)), 16-row MFMA
 * tiles per wave, waves per workgroup, row groups, workgroups in the grid.
 * Passing -plan[1] (or plan[0] when plan[1] == 0) as num_splits to
 * paged_attn_partial reproduces the partial pass of paged_attn_run.
 * Host only; returns PA_EINVAL on a malformed shape. */
int paged_attn_plan(int32_t B, int32_t query_len, int32_t Hq, int32_t Hkv, int32_t D,
                    int32_t page_size, int32_t bt_width, int32_t window, int32_t num_splits,
                    int32_t* plan);

/* Bytes of workspace paged_attn_run needs for this shape (0 when one pass): the
 * fp32 partial outputs and LSEs of S splits, S as paged_attn_resolve_splits
 * resolves num_splits.  It takes the cache geometry (Hkv, page_size, bt_width)
 * and the window because the automatic split count depends on them. */
size_t paged_attn_workspace_size(int32_t B, int32_t query_len, int32_t Hq, int32_t Hkv,
                                 int32_t D, int32_t page_size, int32_t bt_width,
                                 int32_t window, int32_t num_splits);

/* The partial pass of Split-KV alone (fa_utils page: num_splits): for each
 * split s in [0, S) writes the attention restricted to that split's keys.
 * num_splits must be explicit (S >= 1, or -c for chunks of c pages).
 * part_o   [S, B*query_len, Hq, D] fp32, normalized partial outputs.
 * part_lse [S, B*query_len, Hq] fp32 natural-log LSE; -inf marks a split
 *          with no key, whose part_o rows are left unwritten.
 * Other arguments as paged_attn_run. */
int paged_attn_partial(const void* q, int32_t q_dtype, const pa_kv_desc* kv,
                       const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                       const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq,
                       int32_t D, float scale, int32_t window, int32_t num_splits,
                       float* part_o, float* part_lse, hipStream_t stream);

/* Split-KV combine.  For each row r < rows and head h < Hq:
 *   LSE = ln sum_{live s} exp(part_lse[s]);  O = sum_{live s} exp(part_lse[s] - LSE) part_o[s]
 * with live meaning part_lse[s] > -inf; no live split gives O = 0, LSE = -inf.
 * This is the segment combine of the dash_attention page with zero bias.
 * part_o [S, rows, Hq, D] fp32 (dead entries may hold anything, NaN included:
 * they are loaded but never reach the result), part_lse
 * [S, rows, Hq] fp32; out [rows, Hq, D] in out_dtype; lse [rows, Hq] or NULL. */
int split_kv_combine(const float* part_o, const float* part_lse, int32_t S, int32_t rows,
                     int32_t Hq, int32_t D, void* out, int32_t out_dtype, float* lse,
                     hipStream_t stream);

/* DASH segment combine (dash_attention page, flash_dash_attention).
 * For each query n and head h, with prior_g = bias[n, g] for g < G-1 and 0
 * for the last (local) segment, and live_g = used[n, g] > 0:
 *   w = softmax over live g of (part_lse[n, g, h] + prior_g)   (all dead: w = 0)
 *   out[n, h] = sum_{live g} w_g part_o[n, g, h]
 * part_o [N, G, Hq, D] in part_dtype (PA_BF16 | PA_FP16 | PA_F32; dead
 * entries may hold anything: they never reach the result), part_lse
 * [N, G, Hq] fp32, used [N, G] int32,
 * bias [N, G-1] fp32 (may be NULL when G == 1), each finite or -inf: a
 * segment whose logit is -inf weighs nothing, and a query with no finite
 * logit gets out = 0 (the page zeroes the NaN softmax with nan_to_num);
 * out [N, Hq, D] in out_dtype;
 * lse [N, Hq] (logsumexp of the live part_lse + prior, -inf if none) or NULL. */
int segment_attn_combine(const void* part_o, int32_t part_dtype, const float* part_lse,
                         const int32_t* used, const float* bias, int32_t N, int32_t G,
                         int32_t Hq, int32_t D, void* out, int32_t out_dtype, float* lse,
                         hipStream_t stream);

/* DASH segmented attention and its combine (dash_attention page, flash_dash_attention).
 * q [N, Hq, D]; k, v contiguous [N*(topk*bs+local), Hkv, D] in kv_dtype (same
 * 16-bit type as q); per query the rows hold topk remote segments of bs rows
 * and then one local segment of `local` rows.  used [N, topk+1] int32: the
 * number of valid leading rows of each segment (0 = inactive; clamped to the
 * segment's capacity).  bias [N, topk] fp32 (NULL allowed when topk == 0),
 * finite or -inf (a -inf segment weighs nothing, as in segment_attn_combine).
 * Each query attends each segment's valid rows with the given scale (the
 * page uses D**-0.5), then the partial results are merged by
 * segment_attn_combine.  bs and local must be multiples of 8 (PA_EINVAL,
 * as the page requires byte-aligned segments).  The fused path
 * (fused != 0) folds each segment's bias into one online softmax per
 * (query, kv head) and needs no workspace; otherwise the workspace holds the
 * [N, topk+1, Hq, D+1] fp32 partials (segment_attn_workspace_size bytes).
 * out [N, Hq, D] in out_dtype; lse [N, Hq] or NULL.  q, k, v and out are
 * 16-byte aligned; topk <= 63 and N * (topk + 1) < 2^31 (PA_EINVAL otherwise). */
int segment_attn_run(const void* q, int32_t q_dtype, const void* k, const void* v,
                     int32_t kv_dtype, const int32_t* used, const float* bias, int32_t N,
                     int32_t topk, int32_t bs, int32_t local, int32_t Hq, int32_t Hkv,
                     int32_t D, float scale, int32_t fused, void* out, int32_t out_dtype,
                     float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace segment_attn_run needs with fused == 0 (0 for an empty problem). */
size_t segment_attn_workspace_size(int32_t N, int32_t topk, int32_t Hq, int32_t D);

/* Columns of the window-restricted block table (flashinfer_ts, _window_pages):
 * ceil((window + query_len - 1) / page_size) + 1 with a window, bt_width without. */
int32_t paged_attn_window_width(int32_t window, int32_t query_len, int32_t page_size,
                                int32_t bt_width);

/* The integer plan of paged_attn_run, computed on the device by the same code
 * the attention kernels run, so that it can be compared bit-exactly: the
 * window restriction of the flashinfer_ts page (_restrict_to_window: the
 * first visible page, the shortened length, the block table re-based to
 * start there, its columns clamped to the table; _window_pages: the width of
 * that table) and the Split-KV ranges of the fa_utils page (num_splits).
 * Hkv, D and the query shape enter only through the automatic split count:
 *   out_lens  [B]            restricted length L_b - start_page * P
 *   out_table [B, out_width] restricted table: column j = table[b, min(start_page + j, bt_width-1)]
 *                            (out_width = paged_attn_window_width(...)); may be NULL
 *   split_ranges [B, S, 4]   per split: first page (restricted numbering), page
 *                            count, first token, token count; may be NULL
 * num_splits is resolved as in paged_attn_run (S = paged_attn_resolve_splits). */
int paged_attn_describe(const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                        const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq,
                        int32_t Hkv, int32_t D, int32_t page_size, int32_t window,
                        int32_t num_splits, int32_t* out_lens, int32_t* out_table,
                        int32_t out_width, int32_t* split_ranges, hipStream_t stream);

/* paged_attn_describe on HOST memory, by the same inline integer code, with no
 * HIP call (usable without a GPU). */
int paged_attn_describe_host(const int32_t* block_table, int64_t bt_row_stride,
                             int32_t bt_width, const int32_t* seq_lens, int32_t B,
                             int32_t query_len, int32_t Hq, int32_t Hkv, int32_t D,
                             int32_t page_size, int32_t window, int32_t num_splits,
                             int32_t* out_lens, int32_t* out_table, int32_t out_width,
                             int32_t* split_ranges);

/* Paged K/V cache write (flashinfer_ts page, do_kv_cache_update: the new
 * key and value rows of each token go to its slot of the page cache).
 *
 * key, value  [T, Hkv, D] of in_dtype (PA_BF16 | PA_FP16); head rows are
 *             contiguous, tokens key_token_stride / value_token_stride
 *             elements apart (multiples of 16 bytes, >= Hkv*D).
 * slot_mapping [T] int64: token t goes to slot slot_mapping[t] % P of page
 *             slot_mapping[t] / P.  A negative slot (padding) and a slot at
 *             or past num_pages*P write nothing.  Slots of one call must be
 *             distinct (with repeats, which token lands there is unspecified).
 * cache       the pa_kv_desc of the read side; its k and v memory is WRITTEN
 *             (K rows into k, V rows into v, so for vLLM's [pages, Hkv, P, 2D]
 *             page the two halves of each slot row).  dtype = in_dtype (bits
 *             copied) or PA_FP8_E4M3: stored = e4m3fn(x / k_scale) for K and
 *             e4m3fn(x / v_scale) for V, the quotient rounded to fp32, then to
 *             the nearest finite e4m3fn value, ties to even, saturating at
 *             +-448, NaN kept; k_scale, v_scale > 0 and finite.
 * D           multiple of 8 in [8, 256].
 * Async on `stream`; nothing else is read or written.  Errors: PA_ENOTSUP
 * (dtype combination), PA_EINVAL (geometry, strides, alignment, scales,
 * NULL pointers when T > 0), PA_EHIP.  T == 0 is a no-op. */
int paged_kv_write(const void* key, int64_t key_token_stride, const void* value,
                   int64_t value_token_stride, int32_t in_dtype, int32_t T, int32_t D,
                   const int64_t* slot_mapping, const pa_kv_desc* cache, hipStream_t stream);

/* Thread-local message describing the last failing call ("" if none). */
const char* pa_last_error(void);

/* Library version string. */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H_ */
