// Kernel parameter blocks and host launchers shared by the HIP translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum Mode : int {
  MODE_PAGED = 0,          // block-table addressed pages, optional window / Split-KV
  MODE_SEGMENT = 1,        // one work item per (query, segment): partial O / LSE
  MODE_SEGMENT_FUSED = 2,  // one work item per (query, kv head): bias folded, final O
};

struct AttnParams {
  const void* q;        // [items, sq, Hq, D] (segment modes: [N, Hq, D])
  const char* k;        // byte pointers to element 0 of K and V
  const char* v;
  int64_t page_stride;  // elements of the KV type
  int64_t head_stride;
  int64_t token_stride;
  int32_t num_pages;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t bt_width;
  const int32_t* seq_lens;
  int32_t items;        // paged: B; segment: N*(topk+1); fused: N
  int32_t sq, Hq, Hkv, G, R, RG, P, window, S, chunk;
  float qk_scale_log2;  // scale * k_scale * log2(e)
  float v_scale;
  void* out;            // final output (or partial O when S > 1 / segment mode)
  int32_t out_kind;     // K_BF16 | K_FP16 | K_F32
  float* lse;           // may be null unless partial
  int64_t split_stride_o;    // elements between splits of part O (S > 1)
  int64_t split_stride_lse;  // elements between splits of part LSE
  int32_t partial;      // 1: write normalized fp32 partials, skip O of empty items
  const int32_t* used;  // [N, topk+1]
  const float* bias;    // [N, topk]
  int32_t topk, bs, local;
  int32_t window_left;  // causal: keys >= position - window_left (-1: no lower bound)
};

// rows_split = 0: attn_kernel (waves split the keys, RT row tiles per wave);
// rows_split = 1: attn_shared_kernel (paged only; NW waves of one row tile each
// share LDS-staged K/V tiles).
struct LaunchShape {
  int D, kv_kind, q_kind, RT, NW, mode, rows_split;
  int causal;  // paged mode: bottom-right causal rows (exact per-token window)
};

// Rows of attn_kernel's cross-wave merge buffer: a workgroup holds `rows` query
// rows (RT * 16) of which only the first R exist when R is smaller.
__host__ __device__ inline int merge_rows(int R, int rows) { return R < rows ? R : rows; }

// Dynamic LDS bytes of attn_kernel's merge (fp32 O rows padded to D + 4, then m and l).
inline size_t merge_lds_bytes(int D, int NW, int R, int RT) {
  if (NW <= 1) return 0;
  const size_t rr = (size_t)merge_rows(R, RT * 16);
  return (size_t)NW * rr * (size_t)(D + 4) * 4 + 2 * (size_t)NW * rr * 4;
}

// 1 KiB direct-to-LDS loads per staged tile (the shared kernel needs NW to divide it).
int shared_tile_loads(int D, int kv_kind);

hipError_t launch_attention(const AttnParams& p, const LaunchShape& s, int64_t grid,
                            hipStream_t stream);

bool attention_supported(const LaunchShape& s);

// Fused DASH attention with the token rows of kDashHeads kv heads per workgroup
// staged through LDS (dash_shared_kernel): 16-bit K/V, D = 64 or 128, Hq/Hkv <= 16,
// Hkv a multiple of kDashHeads.  One workgroup per (query, head group).
constexpr int kDashHeads = 2;
bool dash_shared_supported(int D, int kv_kind, int G, int Hkv);
hipError_t launch_dash_shared(const AttnParams& p, int D, int kv_kind, hipStream_t stream);

hipError_t launch_split_combine(const float* part_o, const float* part_lse, int32_t S,
                                int32_t rows, int32_t Hq, int32_t D, void* out, int32_t out_kind,
                                float* lse, hipStream_t stream);

hipError_t launch_segment_combine(const void* part_o, int32_t part_kind, const float* part_lse,
                                  const int32_t* used, const float* bias, int32_t N, int32_t G,
                                  int32_t Hq, int32_t D, void* out, int32_t out_kind, float* lse,
                                  hipStream_t stream);

// Paged K/V cache write: token t's rows key[t], value[t] ([Hkv, D] each,
// head-contiguous) into slot slot_mapping[t] of the cache.
struct KVWriteParams {
  const void* key;
  const void* value;
  int64_t key_stride;    // elements between tokens of key
  int64_t value_stride;  // elements between tokens of value
  const int64_t* slot_mapping;
  int32_t T, Hkv, D, P;
  int64_t capacity;      // pages * P
  void* k_cache;
  void* v_cache;
  int64_t page_stride, head_stride, token_stride;  // cache elements
  double k_inv, v_inv;  // fp8 cache: 1 / k_scale, 1 / v_scale rounded to double
};

hipError_t launch_kv_write(const KVWriteParams& p, int in_kind, int cache_kind, hipStream_t stream);

hipError_t launch_describe(const int32_t* block_table, int64_t bt_stride, int32_t bt_width,
                           const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t P,
                           int32_t window, int32_t S, int32_t chunk, int32_t* out_lens,
                           int32_t* out_table, int32_t out_width, int32_t* split_ranges,
                           hipStream_t stream);

}  // namespace pa
