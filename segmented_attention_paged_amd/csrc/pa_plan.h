// Integer plan of the paged-attention path: which keys a request sees and how
// Split-KV cuts them.  The same inline functions run in the attention kernels,
// in the describe kernel and on the host (paged_attn_describe_host), so the
// three agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Visible part of one request after the optional window restriction.
struct SeqView {
  int32_t start_page;  // first visible page of the original table
  int32_t len;         // keys visible, counted from start_page * P
  int32_t n_pages;     // ceil(len / P)
};

// vllm.v1.attention.backends.flashinfer_ts, "Sliding window" / _restrict_to_window:
// the block ends the sequence, so the window is the suffix that starts
// window + query_len - 1 keys before the end, moved down to a page boundary
// and clamped at page 0.  L is first clamped to what the table can address.
__host__ __device__ inline SeqView seq_view(int32_t L, int32_t window, int32_t query_len,
                                            int32_t P, int32_t bt_width) {
  int64_t Lc = L < 0 ? 0 : L;
  const int64_t cap = (int64_t)bt_width * P;
  if (Lc > cap) Lc = cap;
  int64_t sp = 0;
  if (window > 0) {
    const int64_t first = Lc - ((int64_t)window + query_len - 1);
    sp = first > 0 ? first / P : 0;  // non-negative: truncation is the floor
  }
  SeqView v;
  v.start_page = (int32_t)sp;
  v.len = (int32_t)(Lc - sp * P);
  v.n_pages = (int32_t)(v.len > 0 ? cdiv64(v.len, P) : 0);
  return v;
}

// Columns of the restricted table (flashinfer_ts, _window_pages), saturating at
// INT32_MAX for windows of about 2^31 keys over tiny pages.
__host__ __device__ inline int32_t window_width(int32_t window, int32_t query_len, int32_t P,
                                                int32_t bt_width) {
  if (window <= 0) return bt_width;
  const int64_t w = cdiv64((int64_t)window + query_len - 1, P) + 1;
  return (int32_t)(w < INT32_MAX ? w : INT32_MAX);
}

// Column of the caller's table that restricted column j reads (clamped to
// the last column as _restrict_to_window does).
__host__ __device__ inline int32_t table_column(const SeqView& v, int32_t j, int32_t bt_width) {
  const int64_t c = (int64_t)v.start_page + j;
  return (int32_t)(c < bt_width - 1 ? c : bt_width - 1);
}

// One Split-KV chunk in restricted numbering.
struct SplitRange {
  int32_t first_page;
  int32_t n_pages;
  int32_t tok0;
  int32_t n_tok;
};

// chunk > 0: fixed chunks of `chunk` pages; chunk == 0: S chunks of
// ceil(n_pages / S) pages.  Trailing chunks may be empty.
__host__ __device__ inline SplitRange split_range(const SeqView& v, int32_t P, int32_t S,
                                                  int32_t chunk, int32_t s) {
  const int64_t per = chunk > 0 ? chunk : (v.n_pages > 0 ? cdiv64(v.n_pages, S) : 0);
  int64_t first = (int64_t)s * per;
  int64_t last = first + per;
  if (first > v.n_pages) first = v.n_pages;
  if (last > v.n_pages) last = v.n_pages;
  SplitRange r;
  r.first_page = (int32_t)first;
  r.n_pages = (int32_t)(last - first);
  const int64_t t0 = first * P;
  int64_t t1 = last * P;
  if (t1 > v.len) t1 = v.len;
  r.tok0 = (int32_t)t0;
  r.n_tok = (int32_t)(t1 > t0 ? t1 - t0 : 0);
  return r;
}

// Library split policy for num_splits: S > 0 explicit; -c fixed chunks of
// c pages; 0 automatic.  `pages_max` is the static bound on visible pages.
struct SplitPolicy {
  int32_t S;
  int32_t chunk;  // 0: ceil(n / S) pages per split
};

__host__ __device__ inline int32_t pages_bound(int32_t window, int32_t query_len, int32_t P,
                                               int32_t bt_width) {
  if (window <= 0) return bt_width;
  const int32_t w = window_width(window, query_len, P, bt_width);
  return w < bt_width ? w : bt_width;
}

}  // namespace pa
