// C ABI of the paged-attention library: argument checks, split planning,
// workspace carving and kernel dispatch.  Host code (plus the device scratch
// array of the allocation-free entry point); it never allocates, synchronizes
// or reads device memory, so every entry point can be captured into a hipGraph.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/paged_attn.h"
#include "pa_kernels.h"
#include "pa_plan.h"

// Waves per workgroup of attn_kernel's segment modes at one 16-row tile per
// wave: the fused mode (odd Hkv, or more than 16 query heads per kv head; the
// rest go to dash_shared_kernel) splits a (query, kv head)'s tiles over 4
// waves; the two-stage kernel's items (one segment) are a few tiles long and
// take one wave.
constexpr int kSegFusedWaves = 4;
constexpr int kSegWaves = 1;

using namespace pa;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return PA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kTargetWorkgroups = 2048;  // workgroups the automatic split aims for

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

struct Plan {
  int RT, NW, RG;
  int S, chunk;
  int rows_split;
};

// Up to 16 rows (decode): 4 waves split the keys of a work item.  More rows
// (query blocks): one 16-row tile per wave, the waves sharing LDS-staged K/V
// tiles; at most as many waves as a staged tile has 1 KiB loads for fp8 K/V
// of this head_dim (so the plan does not depend on the cache dtype).
Plan make_plan(int32_t B, int32_t sq, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
               int32_t bt_width, int32_t window, int32_t num_splits) {
  Plan pl{};
  const int G = Hq / Hkv;
  const int R = G * sq;
  if (R <= 16) {
    pl.rows_split = 0;
    pl.RT = 1;
    pl.NW = 4;
    pl.RG = 1;
  } else {
    pl.rows_split = 1;
    pl.RT = 1;
    const int max_nw = std::min(8, shared_tile_loads(D, PA_FP8_E4M3));
    int nw = 2;
    while (nw < max_nw && 16 * nw < R) nw *= 2;
    pl.NW = nw;
    pl.RG = (int)cdiv(R, 16 * nw);
  }
  const int32_t pages_max = pages_bound(window, sq, P, bt_width);
  if (num_splits > 0) {
    pl.S = num_splits;
    pl.chunk = 0;
  } else if (num_splits < 0) {
    pl.chunk = -num_splits;
    pl.S = (int)std::max<int64_t>(1, cdiv(pages_max, pl.chunk));
    if (pl.S == 1) pl.chunk = 0;
  } else {
    // A few equal splits per request: enough workgroups to fill the chip, few
    // enough that the per-workgroup start-up and the partial round trip stay
    // small.  The partials of the row-split kernel (query blocks) are R rows
    // per item, so it takes fewer, longer splits.
    const int64_t items = (int64_t)B * Hkv * pl.RG;
    int64_t S = cdiv(kTargetWorkgroups, std::max<int64_t>(items, 1));
    // at least 16 tiles per split (64 for the row-split kernel) so start-up
    // and the partial write stay amortized
    const int64_t min_tiles = pl.rows_split ? 64 : 16;
    const int64_t min_pages_per_split = std::max<int64_t>(1, cdiv(min_tiles, cdiv(P, 16)));
    S = std::min<int64_t>(S, std::max<int64_t>(1, pages_max / min_pages_per_split));
    S = std::max<int64_t>(1, std::min<int64_t>(S, 64));
    pl.S = (int)S;
    pl.chunk = 0;
  }
  return pl;
}

int kind_bytes(int kind) { return kind == PA_F32 ? 4 : (kind == PA_FP8_E4M3 ? 1 : 2); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by paged_attn_run / paged_attn_partial.
int check_paged(const void* q, int32_t q_dtype, const pa_kv_desc* kv, const int32_t* block_table,
                int64_t bt_row_stride, int32_t bt_width, const int32_t* seq_lens, int32_t B,
                int32_t query_len, int32_t Hq, int32_t D, float scale) {
  if (B < 0 || query_len < 0) return fail(PA_EINVAL, "B and query_len must be >= 0");
  if (!kv) return fail(PA_EINVAL, "kv descriptor is NULL");
  if (q_dtype != PA_BF16 && q_dtype != PA_FP16 && q_dtype != PA_FP8_E4M3)
    return fail(PA_ENOTSUP, "query dtype must be bf16, fp16 or fp8_e4m3 (got %d)", q_dtype);
  if (kv->dtype != PA_BF16 && kv->dtype != PA_FP16 && kv->dtype != PA_FP8_E4M3)
    return fail(PA_ENOTSUP, "kv dtype must be bf16, fp16 or fp8_e4m3 (got %d)", kv->dtype);
  if (kv->dtype != PA_FP8_E4M3 && kv->dtype != q_dtype)
    return fail(PA_ENOTSUP, "a 16-bit cache needs a query of the same dtype");
  if (q_dtype == PA_FP8_E4M3 && kv->dtype != PA_FP8_E4M3)
    return fail(PA_ENOTSUP, "an fp8 query needs an fp8 cache");
  if (D != 64 && D != 128) return fail(PA_EINVAL, "head_dim must be 64 or 128 (got %d)", D);
  if (Hq <= 0 || kv->num_kv_heads <= 0 || Hq % kv->num_kv_heads)
    return fail(PA_EINVAL, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, kv->num_kv_heads);
  if (kv->page_size < 1 || kv->page_size > (1 << 20)) return fail(PA_EINVAL, "page_size out of range");
  if (kv->num_pages < 1) return fail(PA_EINVAL, "num_pages must be >= 1");
  if (bt_width < 1 || bt_row_stride < bt_width) return fail(PA_EINVAL, "bad block-table shape");
  if (!(std::isfinite(scale))) return fail(PA_EINVAL, "scale must be finite");
  if (kv->dtype == PA_FP8_E4M3 &&
      !(kv->k_scale > 0.f && kv->v_scale > 0.f && std::isfinite(kv->k_scale) && std::isfinite(kv->v_scale)))
    return fail(PA_EINVAL, "fp8 cache needs positive finite k_scale and v_scale");
  if (!(std::isfinite(kv->k_scale) && std::isfinite(kv->v_scale)))
    return fail(PA_EINVAL, "k_scale and v_scale must be finite");
  const int eb = kind_bytes(kv->dtype);
  if ((kv->page_stride * eb) % 16 || (kv->head_stride * eb) % 16 || (kv->token_stride * eb) % 16 ||
      kv->page_stride < 0 || kv->head_stride < 0 || kv->token_stride <= 0)
    return fail(PA_EINVAL, "kv strides must be non-negative multiples of 16 bytes");
  if (kv->token_stride * eb > (int64_t)1 << 26)  // lane offsets inside a tile are 32-bit
    return fail(PA_EINVAL, "token stride above 64 MiB");
  // query rows (B*query_len) and rows per kv head ((Hq/Hkv)*query_len) are 32-bit counts
  if ((int64_t)B * query_len > INT32_MAX || (int64_t)(Hq / kv->num_kv_heads) * query_len > INT32_MAX)
    return fail(PA_EINVAL, "B*query_len and (Hq/Hkv)*query_len must be below 2^31");
  if (B == 0 || query_len == 0) return PA_OK;
  if (!q || !kv->k || !kv->v || !block_table || !seq_lens)
    return fail(PA_EINVAL, "NULL input pointer");
  if (!aligned16(q) || !aligned16(kv->k) || !aligned16(kv->v))
    return fail(PA_EINVAL, "q, k and v must be 16-byte aligned");
  return PA_OK;
}

AttnParams paged_params(const void* q, const pa_kv_desc* kv, const int32_t* block_table,
                        int64_t bt_row_stride, int32_t bt_width, const int32_t* seq_lens, int32_t B,
                        int32_t query_len, int32_t Hq, float scale, int32_t window,
                        const Plan& pl) {
  AttnParams p{};
  p.q = q;
  p.k = static_cast<const char*>(kv->k);
  p.v = static_cast<const char*>(kv->v);
  p.page_stride = kv->page_stride;
  p.head_stride = kv->head_stride;
  p.token_stride = kv->token_stride;
  p.num_pages = kv->num_pages;
  p.block_table = block_table;
  p.bt_stride = bt_row_stride;
  p.bt_width = bt_width;
  p.seq_lens = seq_lens;
  p.items = B;
  p.sq = query_len;
  p.Hq = Hq;
  p.Hkv = kv->num_kv_heads;
  p.G = Hq / kv->num_kv_heads;
  p.R = p.G * query_len;
  p.RG = pl.RG;
  p.P = kv->page_size;
  p.window = window > 0 ? window : 0;
  p.S = pl.S;
  p.chunk = pl.chunk;
  p.qk_scale_log2 = scale * kv->k_scale * 1.4426950408889634f;
  p.v_scale = kv->v_scale;
  return p;
}

}  // namespace

// ---- allocation-free variant of paged_attn_run ------------------------------------
// The Split-KV partials of paged_attn_run_noalloc live in this file-scope device
// array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy (at its own address) until the process ends.  In host code the name
// `scratch` is only a host-side stand-in: its device address is looked up once
// per device with hipGetSymbolAddress and only that address is used.
static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device `stream` belongs to (the current
// device for the null stream), looked up on the first call for that device
// with that device current.
int scratch_for_stream(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ENOTSUP, "device %d: the allocation-free scratch covers devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) return hip_fail(e2, "hipSetDevice");
    }
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(PA_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}
}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_err; }

const char* pa_version(void) { return "segmented_attention_paged_amd 0.1 (gfx950)"; }

int32_t paged_attn_window_width(int32_t window, int32_t query_len, int32_t page_size,
                                int32_t bt_width) {
  if (page_size < 1) return 0;
  return window_width(window, query_len, page_size, bt_width);
}

int32_t paged_attn_resolve_splits(int32_t B, int32_t query_len, int32_t Hq, int32_t Hkv,
                                  int32_t D, int32_t page_size, int32_t bt_width, int32_t window,
                                  int32_t num_splits) {
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv || page_size < 1 || bt_width < 1 || query_len < 1) return 1;
  return make_plan(B, query_len, Hq, Hkv, D, page_size, bt_width, window, num_splits).S;
}

int paged_attn_plan(int32_t B, int32_t query_len, int32_t Hq, int32_t Hkv, int32_t D,
                    int32_t page_size, int32_t bt_width, int32_t window, int32_t num_splits,
                    int32_t* plan) {
  if (!plan) return fail(PA_EINVAL, "plan is NULL");
  if (B < 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || page_size < 1 || bt_width < 1 || query_len < 1)
    return fail(PA_EINVAL, "bad plan geometry");
  const Plan pl = make_plan(B, query_len, Hq, Hkv, D, page_size, bt_width, window, num_splits);
  plan[0] = pl.S;
  plan[1] = pl.chunk;
  plan[2] = pl.RT;
  plan[3] = pl.NW;
  plan[4] = pl.RG;
  plan[5] = (int32_t)std::min<int64_t>((int64_t)B * Hkv * pl.RG * pl.S, 0x7fffffff);
  return ok();
}

size_t paged_attn_workspace_size(int32_t B, int32_t query_len, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t page_size, int32_t bt_width, int32_t window,
                                 int32_t num_splits) {
  const int32_t S =
      paged_attn_resolve_splits(B, query_len, Hq, Hkv, D, page_size, bt_width, window, num_splits);
  if (S <= 1 || B <= 0 || query_len <= 0) return 0;
  const int64_t rows = (int64_t)B * query_len * Hq;
  return (size_t)(align256((int64_t)S * rows * D * 4) + align256((int64_t)S * rows * 4));
}

// The partial pass of Split-KV (or the whole attention when S == 1 and `out`
// is final) for one resolved plan.
static int launch_paged(const void* q, int32_t q_dtype, const pa_kv_desc* kv,
                        const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                        const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq,
                        int32_t D, float scale, int32_t window, const Plan& pl, void* out,
                        int32_t out_kind, float* lse, bool partial, hipStream_t stream,
                        bool causal = false) {
  AttnParams p = paged_params(q, kv, block_table, bt_row_stride, bt_width, seq_lens, B, query_len,
                              Hq, scale, window, pl);
  // causal: the page restriction of the window only skips pages no token can
  // reach; the kernel applies the exact per-token window of `window` keys
  p.window_left = (causal && window > 0) ? window - 1 : -1;
  const int64_t rows = (int64_t)B * query_len * Hq;
  p.out = out;
  p.out_kind = out_kind;
  p.lse = lse;
  p.partial = partial ? 1 : 0;
  p.split_stride_o = rows * D;
  p.split_stride_lse = rows;
  LaunchShape ls{D, kv->dtype, q_dtype, pl.RT, pl.NW, MODE_PAGED, pl.rows_split, causal ? 1 : 0};
  if (pl.rows_split && (shared_tile_loads(D, kv->dtype) % pl.NW) != 0)
    return fail(PA_ENOTSUP, "no shared-tile kernel for this head_dim / dtype / wave count");
  const int64_t grid = (int64_t)B * kv->num_kv_heads * pl.RG * pl.S;
  hipError_t e = launch_attention(p, ls, grid, stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return PA_OK;
}

int paged_attn_partial(const void* q, int32_t q_dtype, const pa_kv_desc* kv,
                       const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                       const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq, int32_t D,
                       float scale, int32_t window, int32_t num_splits, float* part_o,
                       float* part_lse, hipStream_t stream) {
  int rc = check_paged(q, q_dtype, kv, block_table, bt_row_stride, bt_width, seq_lens, B, query_len,
                       Hq, D, scale);
  if (rc != PA_OK) return rc;
  if (num_splits == 0) return fail(PA_EINVAL, "paged_attn_partial needs an explicit num_splits");
  if (B == 0 || query_len == 0) return ok();
  if (!part_o || !part_lse || !aligned16(part_o)) return fail(PA_EINVAL, "bad partial buffers");
  const Plan pl = make_plan(B, query_len, Hq, kv->num_kv_heads, D, kv->page_size, bt_width, window,
                            num_splits);
  rc = launch_paged(q, q_dtype, kv, block_table, bt_row_stride, bt_width, seq_lens, B, query_len, Hq,
                    D, scale, window, pl, part_o, PA_F32, part_lse, true, stream);
  return rc == PA_OK ? ok() : rc;
}

static int run_paged(const void* q, int32_t q_dtype, const pa_kv_desc* kv,
                     const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                     const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq, int32_t D,
                     float scale, int32_t window, int32_t num_splits, void* out, int32_t out_dtype,
                     float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream,
                     bool causal) {
  int rc = check_paged(q, q_dtype, kv, block_table, bt_row_stride, bt_width, seq_lens, B, query_len,
                       Hq, D, scale);
  if (rc != PA_OK) return rc;
  if (out_dtype != PA_BF16 && out_dtype != PA_FP16 && out_dtype != PA_F32)
    return fail(PA_ENOTSUP, "out dtype must be bf16, fp16 or f32 (got %d)", out_dtype);
  if (B == 0 || query_len == 0) return ok();
  if (!out || !aligned16(out)) return fail(PA_EINVAL, "out must be a 16-byte aligned pointer");
  const Plan pl = make_plan(B, query_len, Hq, kv->num_kv_heads, D, kv->page_size, bt_width, window,
                            num_splits);
  if (pl.S == 1) {
    rc = launch_paged(q, q_dtype, kv, block_table, bt_row_stride, bt_width, seq_lens, B, query_len,
                      Hq, D, scale, window, pl, out, out_dtype, lse, false, stream, causal);
    return rc == PA_OK ? ok() : rc;
  }
  const size_t need = paged_attn_workspace_size(B, query_len, Hq, kv->num_kv_heads, D,
                                                kv->page_size, bt_width, window, num_splits);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(PA_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  const int64_t rows = (int64_t)B * query_len * Hq;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             align256((int64_t)pl.S * rows * D * 4));
  rc = launch_paged(q, q_dtype, kv, block_table, bt_row_stride, bt_width, seq_lens, B, query_len, Hq,
                    D, scale, window, pl, part_o, PA_F32, part_lse, true, stream, causal);
  if (rc != PA_OK) return rc;
  hipError_t e = launch_split_combine(part_o, part_lse, pl.S, (int32_t)(B * query_len), Hq, D, out,
                                      out_dtype, lse, stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

int paged_attn_run(const void* q, int32_t q_dtype, const pa_kv_desc* kv,
                   const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                   const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq, int32_t D,
                   float scale, int32_t window, int32_t num_splits, void* out, int32_t out_dtype,
                   float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_paged(q, q_dtype, kv, block_table, bt_row_stride, bt_width, seq_lens, B, query_len, Hq,
                   D, scale, window, num_splits, out, out_dtype, lse, workspace, workspace_bytes,
                   stream, false);
}

int paged_attn_run_noalloc(const void* q, int32_t q_dtype, const pa_kv_desc* kv,
                           const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                           const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq,
                           int32_t D, float scale, int32_t window, int32_t num_splits, void* out,
                           int32_t out_dtype, float* lse, hipStream_t stream) {
  int rc = check_paged(q, q_dtype, kv, block_table, bt_row_stride, bt_width, seq_lens, B, query_len,
                       Hq, D, scale);
  if (rc != PA_OK) return rc;
  if (B == 0 || query_len == 0) return ok();
  const size_t need = paged_attn_workspace_size(B, query_len, Hq, kv->num_kv_heads, D,
                                                kv->page_size, bt_width, window, num_splits);
  void* ws = nullptr;
  if (need > 0) {
    if (need > PA_NOALLOC_SCRATCH_BYTES)
      return fail(PA_EWORKSPACE,
                  "paged_attn_run_noalloc: this shape needs %zu bytes of Split-KV partials, more "
                  "than its %zu-byte scratch; use paged_attn_run with a workspace or fewer splits",
                  need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
    rc = scratch_for_stream(stream, &ws);
    if (rc != PA_OK) return rc;
  }
  return run_paged(q, q_dtype, kv, block_table, bt_row_stride, bt_width, seq_lens, B, query_len, Hq,
                   D, scale, window, num_splits, out, out_dtype, lse, ws, need, stream, false);
}

int paged_attn_run_causal(const void* q, int32_t q_dtype, const pa_kv_desc* kv,
                          const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                          const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq,
                          int32_t D, float scale, int32_t window, int32_t num_splits, void* out,
                          int32_t out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return run_paged(q, q_dtype, kv, block_table, bt_row_stride, bt_width, seq_lens, B, query_len, Hq,
                   D, scale, window, num_splits, out, out_dtype, lse, workspace, workspace_bytes,
                   stream, true);
}

int split_kv_combine(const float* part_o, const float* part_lse, int32_t S, int32_t rows,
                     int32_t Hq, int32_t D, void* out, int32_t out_dtype, float* lse,
                     hipStream_t stream) {
  if (S < 1 || rows < 0 || Hq < 0) return fail(PA_EINVAL, "bad combine shape");
  if (D < 1 || D > 256) return fail(PA_EINVAL, "head_dim must be in [1, 256]");
  if (out_dtype != PA_BF16 && out_dtype != PA_FP16 && out_dtype != PA_F32)
    return fail(PA_ENOTSUP, "out dtype must be bf16, fp16 or f32");
  if (rows == 0 || Hq == 0) return ok();
  if (!part_o || !part_lse || !out) return fail(PA_EINVAL, "NULL pointer");
  hipError_t e = launch_split_combine(part_o, part_lse, S, rows, Hq, D, out, out_dtype, lse, stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

int segment_attn_combine(const void* part_o, int32_t part_dtype, const float* part_lse,
                         const int32_t* used, const float* bias, int32_t N, int32_t G, int32_t Hq,
                         int32_t D, void* out, int32_t out_dtype, float* lse, hipStream_t stream) {
  if (N < 0 || G < 1 || Hq < 0) return fail(PA_EINVAL, "bad combine shape");
  if (D < 1 || D > 256) return fail(PA_EINVAL, "head_dim must be in [1, 256]");
  if (part_dtype != PA_BF16 && part_dtype != PA_FP16 && part_dtype != PA_F32)
    return fail(PA_ENOTSUP, "partial dtype must be bf16, fp16 or f32");
  if (out_dtype != PA_BF16 && out_dtype != PA_FP16 && out_dtype != PA_F32)
    return fail(PA_ENOTSUP, "out dtype must be bf16, fp16 or f32");
  if (N == 0 || Hq == 0) return ok();
  if (!part_o || !part_lse || !used || !out || (G > 1 && !bias))
    return fail(PA_EINVAL, "NULL pointer");
  hipError_t e = launch_segment_combine(part_o, part_dtype, part_lse, used, bias, N, G, Hq, D, out,
                                        out_dtype, lse, stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

size_t segment_attn_workspace_size(int32_t N, int32_t topk, int32_t Hq, int32_t D) {
  if (N <= 0 || topk < 0 || Hq <= 0 || D <= 0) return 0;
  const int64_t rows = (int64_t)N * (topk + 1) * Hq;
  return (size_t)(align256(rows * D * 4) + align256(rows * 4));
}

int segment_attn_run(const void* q, int32_t q_dtype, const void* k, const void* v,
                     int32_t kv_dtype, const int32_t* used, const float* bias, int32_t N,
                     int32_t topk, int32_t bs, int32_t local, int32_t Hq, int32_t Hkv, int32_t D,
                     float scale, int32_t fused, void* out, int32_t out_dtype, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (q_dtype != PA_BF16 && q_dtype != PA_FP16)
    return fail(PA_ENOTSUP, "segment attention needs a bf16 or fp16 query (got %d)", q_dtype);
  if (kv_dtype != q_dtype) return fail(PA_ENOTSUP, "segment K/V must have the query's dtype");
  if (bs % 8 || local % 8 || bs < 0 || local < 0)
    return fail(PA_EINVAL, "segments must be multiples of 8 rows (bs=%d, local=%d)", bs, local);
  if (N < 0 || topk < 0 || topk > 63) return fail(PA_EINVAL, "bad N or topk");
  if ((int64_t)N * (topk + 1) > INT32_MAX) return fail(PA_EINVAL, "N*(topk+1) must be below 2^31");
  if (D != 64 && D != 128) return fail(PA_EINVAL, "head_dim must be 64 or 128");
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv) return fail(PA_EINVAL, "Hq must be a positive multiple of Hkv");
  if ((int64_t)Hkv * D * 2 > (int64_t)1 << 26) return fail(PA_EINVAL, "token stride above 64 MiB");
  if (out_dtype != PA_BF16 && out_dtype != PA_FP16 && out_dtype != PA_F32)
    return fail(PA_ENOTSUP, "out dtype must be bf16, fp16 or f32");
  if (!std::isfinite(scale)) return fail(PA_EINVAL, "scale must be finite");
  if (N == 0) return ok();
  if (!q || !k || !v || !used || !out || (topk > 0 && !bias)) return fail(PA_EINVAL, "NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(PA_EINVAL, "q, k, v and out must be 16-byte aligned");
  const int G = Hq / Hkv;
  const int R = G;  // one query token
  const int RT = R <= 16 ? 1 : (R <= 32 ? 2 : 4);
  const int RG = (int)cdiv(R, 16 * RT);
  AttnParams p{};
  p.q = q;
  p.k = static_cast<const char*>(k);
  p.v = static_cast<const char*>(v);
  p.token_stride = (int64_t)Hkv * D;
  p.head_stride = D;
  p.page_stride = 0;
  p.sq = 1;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = G;
  p.R = R;
  p.RG = RG;
  p.S = 1;
  p.qk_scale_log2 = scale * 1.4426950408889634f;
  p.v_scale = 1.f;
  p.used = used;
  p.bias = bias;
  p.topk = topk;
  p.bs = bs;
  p.local = local;
  if (fused) {
    const int NW = RT == 1 ? kSegFusedWaves : 4 / RT;
    p.items = N;
    p.out = out;
    p.out_kind = out_dtype;
    p.lse = lse;
    p.partial = 0;
    if (dash_shared_supported(D, kv_dtype, G, Hkv)) {
      hipError_t e = launch_dash_shared(p, D, kv_dtype, stream);
      if (e != hipSuccess) return hip_fail(e, "segment attention launch");
      return ok();
    }
    const LaunchShape ls{D, kv_dtype, q_dtype, RT, NW, MODE_SEGMENT_FUSED, 0, 0};
    hipError_t e = launch_attention(p, ls, (int64_t)N * Hkv * RG, stream);
    if (e != hipSuccess) return hip_fail(e, "segment attention launch");
    return ok();
  }
  const size_t need = segment_attn_workspace_size(N, topk, Hq, D);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(PA_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  const int Gs = topk + 1;
  const int64_t rows = (int64_t)N * Gs * Hq;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(rows * D * 4));
  const int NW = RT == 1 ? kSegWaves : 4 / RT;
  p.out = part_o;
  p.out_kind = PA_F32;
  p.lse = part_lse;
  p.partial = 1;
  hipError_t e;
  if (dash_shared_supported(D, kv_dtype, G, Hkv)) {
    p.items = N;  // one workgroup per (query, kv-head group) walks all its segments
    e = launch_dash_shared(p, D, kv_dtype, stream);
  } else {
    p.items = N * Gs;
    const LaunchShape ls{D, kv_dtype, q_dtype, RT, NW, MODE_SEGMENT, 0, 0};
    e = launch_attention(p, ls, (int64_t)N * Gs * Hkv * RG, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "segment attention launch");
  e = launch_segment_combine(part_o, PA_F32, part_lse, used, bias, N, Gs, Hq, D, out, out_dtype,
                             lse, stream);
  if (e != hipSuccess) return hip_fail(e, "segment combine launch");
  return ok();
}

static int describe_checks(int32_t bt_width, int64_t bt_row_stride, int32_t B, int32_t query_len,
                           int32_t Hq, int32_t Hkv, int32_t page_size) {
  if (B < 0 || query_len < 1 || page_size < 1 || bt_width < 1 || bt_row_stride < bt_width)
    return fail(PA_EINVAL, "bad describe geometry");
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv) return fail(PA_EINVAL, "Hq must be a positive multiple of Hkv");
  return PA_OK;
}

int paged_attn_describe(const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                        const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq,
                        int32_t Hkv, int32_t D, int32_t page_size, int32_t window,
                        int32_t num_splits, int32_t* out_lens, int32_t* out_table,
                        int32_t out_width, int32_t* split_ranges, hipStream_t stream) {
  (void)D;
  int rc = describe_checks(bt_width, bt_row_stride, B, query_len, Hq, Hkv, page_size);
  if (rc != PA_OK) return rc;
  if (B == 0) return ok();
  if (!block_table || !seq_lens || !out_lens) return fail(PA_EINVAL, "NULL pointer");
  const Plan pl = make_plan(B, query_len, Hq, Hkv, D, page_size, bt_width, window, num_splits);
  hipError_t e = launch_describe(block_table, bt_row_stride, bt_width, seq_lens, B, query_len,
                                 page_size, window > 0 ? window : 0, pl.S, pl.chunk, out_lens,
                                 out_table, out_width, split_ranges, stream);
  if (e != hipSuccess) return hip_fail(e, "describe launch");
  return ok();
}

int paged_attn_describe_host(const int32_t* block_table, int64_t bt_row_stride, int32_t bt_width,
                             const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t Hq,
                             int32_t Hkv, int32_t D, int32_t page_size, int32_t window,
                             int32_t num_splits, int32_t* out_lens, int32_t* out_table,
                             int32_t out_width, int32_t* split_ranges) {
  (void)D;
  int rc = describe_checks(bt_width, bt_row_stride, B, query_len, Hq, Hkv, page_size);
  if (rc != PA_OK) return rc;
  if (B == 0) return ok();
  if (!block_table || !seq_lens || !out_lens) return fail(PA_EINVAL, "NULL pointer");
  const Plan pl = make_plan(B, query_len, Hq, Hkv, D, page_size, bt_width, window, num_splits);
  const int32_t w = window > 0 ? window : 0;
  for (int b = 0; b < B; ++b) {
    const SeqView sv = seq_view(seq_lens[b], w, query_len, page_size, bt_width);
    out_lens[b] = sv.len;
    if (out_table)
      for (int j = 0; j < out_width; ++j)
        out_table[(int64_t)b * out_width + j] =
            block_table[(int64_t)b * bt_row_stride + table_column(sv, j, bt_width)];
    if (split_ranges)
      for (int s = 0; s < pl.S; ++s) {
        const SplitRange r = split_range(sv, page_size, pl.S, pl.chunk, s);
        int32_t* o = split_ranges + ((int64_t)b * pl.S + s) * 4;
        o[0] = r.first_page;
        o[1] = r.n_pages;
        o[2] = r.tok0;
        o[3] = r.n_tok;
      }
  }
  return ok();
}

int paged_kv_write(const void* key, int64_t key_token_stride, const void* value,
                   int64_t value_token_stride, int32_t in_dtype, int32_t T, int32_t D,
                   const int64_t* slot_mapping, const pa_kv_desc* cache, hipStream_t stream) {
  if (!cache) return fail(PA_EINVAL, "cache descriptor is NULL");
  if (in_dtype != PA_BF16 && in_dtype != PA_FP16)
    return fail(PA_ENOTSUP, "key/value dtype must be bf16 or fp16 (got %d)", in_dtype);
  if (cache->dtype != in_dtype && cache->dtype != PA_FP8_E4M3)
    return fail(PA_ENOTSUP, "cache dtype must be the input's or fp8_e4m3 (got %d)", cache->dtype);
  if (T < 0) return fail(PA_EINVAL, "T must be >= 0");
  if (D < 8 || D > 256 || D % 8) return fail(PA_EINVAL, "head_dim must be a multiple of 8 in [8, 256]");
  const int32_t Hkv = cache->num_kv_heads, P = cache->page_size;
  if (Hkv <= 0 || P <= 0 || cache->num_pages < 0) return fail(PA_EINVAL, "bad cache geometry");
  if (key_token_stride < (int64_t)Hkv * D || value_token_stride < (int64_t)Hkv * D ||
      (key_token_stride * 2) % 16 || (value_token_stride * 2) % 16)
    return fail(PA_EINVAL, "key/value token strides must cover Hkv*D values and be multiples of 16 bytes");
  const int eb = kind_bytes(cache->dtype);
  if ((cache->page_stride * eb) % 16 || (cache->head_stride * eb) % 16 || (cache->token_stride * eb) % 16 ||
      cache->page_stride < 0 || cache->head_stride < 0 || cache->token_stride <= 0)
    return fail(PA_EINVAL, "cache strides must be non-negative multiples of 16 bytes");
  if (cache->dtype == PA_FP8_E4M3 &&
      !(cache->k_scale > 0.f && cache->v_scale > 0.f && std::isfinite(cache->k_scale) &&
        std::isfinite(cache->v_scale)))
    return fail(PA_EINVAL, "fp8 cache needs positive finite k_scale and v_scale");
  if (T == 0 || cache->num_pages == 0) return ok();
  if (!key || !value || !slot_mapping || !cache->k || !cache->v) return fail(PA_EINVAL, "NULL pointer");
  if (!aligned16(key) || !aligned16(value) || !aligned16(cache->k) || !aligned16(cache->v))
    return fail(PA_EINVAL, "key, value and the cache must be 16-byte aligned");
  KVWriteParams p{};
  p.key = key;
  p.value = value;
  p.key_stride = key_token_stride;
  p.value_stride = value_token_stride;
  p.slot_mapping = slot_mapping;
  p.T = T;
  p.Hkv = Hkv;
  p.D = D;
  p.P = P;
  p.capacity = (int64_t)cache->num_pages * P;
  p.k_cache = const_cast<void*>(cache->k);
  p.v_cache = const_cast<void*>(cache->v);
  p.page_stride = cache->page_stride;
  p.head_stride = cache->head_stride;
  p.token_stride = cache->token_stride;
  p.k_inv = 1.0 / (double)cache->k_scale;
  p.v_inv = 1.0 / (double)cache->v_scale;
  hipError_t e = launch_kv_write(p, in_dtype, cache->dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "cache write launch");
  return ok();
}

}  // extern "C"
