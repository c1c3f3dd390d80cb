// LSE-weighted combine kernels (Split-KV partials, DASH segments) and the
// device-side integer plan dump.
//
// Both combines are the merge that closes flash_dash_attention on the
// vllm.v1.attention.ops.dash_attention page: logits = partial LSE + prior,
// softmax over the live partials (dead ones excluded, all-dead giving zero
// weights), output = weighted sum of the live partial outputs.  Split-KV uses
// it with a zero prior and "live" meaning a finite partial LSE.
//
// One wave per (row, head).  Lane s holds the logit of partial s; lanes own
// head-dim columns d = lane + 64c.  Partial rows are fetched in batches of 8
// independent loads per lane, issued without waiting for the logits, and a
// dead partial's row (possibly never written) only ever meets a select, so it
// cannot leak into the result.

#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_plan.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kBatch = 8;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int PK>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
  if constexpr (PK == K_F32) return reinterpret_cast<const float*>(base)[i];
  const uint16_t b = reinterpret_cast<const uint16_t*>(base)[i];
  if constexpr (PK == K_BF16) return __uint_as_float((uint32_t)b << 16);
  return (float)bitcast<_Float16>(b);
}

__device__ __forceinline__ void store_elem(void* base, int64_t i, int kind, float x) {
  if (kind == K_F32) {
    reinterpret_cast<float*>(base)[i] = x;
  } else if (kind == K_BF16) {
    reinterpret_cast<__bf16*>(base)[i] = (__bf16)x;
  } else {
    reinterpret_cast<_Float16*>(base)[i] = (_Float16)x;
  }
}

// Merge G partial rows (row g at obase + g * ostride, element kind PK) of one
// (row, head).  `logit(g)` is the natural-log logit of partial g, -inf if dead.
// C = ceil(D / 64) head-dim columns per lane.
template <int C, int PK, typename LogitFn>
__device__ __forceinline__ void merge_row(int G, int D, LogitFn logit, const void* obase,
                                          int64_t ostride, void* out, int64_t out_off,
                                          int out_kind, float* lse, int64_t lse_off) {
  const int lane = threadIdx.x & 63;
  float M = kNegInf;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    M = fmaxf(M, g < G ? logit(g) : kNegInf);
  }
  M = wave_max(M);
  float o[C];
#pragma unroll
  for (int c = 0; c < C; ++c) o[c] = 0.f;
  float tot = 0.f;
  if (M != kNegInf) {
    for (int g0 = 0; g0 < G; g0 += 64) {
      const int g = g0 + lane;
      const float lg = g < G ? logit(g) : kNegInf;
      const float w_lane = lg == kNegInf ? 0.f : fast_exp2((lg - M) * kLog2e);
      tot += w_lane;
      const int n = G - g0 < 64 ? G - g0 : 64;
      for (int j = 0; j < n; j += kBatch) {
        float x[kBatch][C];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int gg = g0 + (j + u < n ? j + u : 0);
#pragma unroll
          for (int c = 0; c < C; ++c) {
            const int d = lane + 64 * c;
            x[u][c] = d < D ? load_elem<PK>(obase, (int64_t)gg * ostride + d) : 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float w = __shfl(w_lane, j + u < n ? j + u : 0, 64);
          const bool use = (j + u < n) && w > 0.f;
#pragma unroll
          for (int c = 0; c < C; ++c) o[c] = use ? o[c] + w * x[u][c] : o[c];
        }
      }
    }
    tot = wave_sum(tot);
    const float inv = 1.f / tot;
#pragma unroll
    for (int c = 0; c < C; ++c) o[c] *= inv;
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int d = lane + 64 * c;
    if (d < D) store_elem(out, out_off + d, out_kind, o[c]);
  }
  if (lse && lane == 0) lse[lse_off] = tot > 0.f ? M + logf(tot) : kNegInf;
}

template <int C>
__global__ __launch_bounds__(256) void split_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_lse,
                                                            int32_t S, int32_t rows, int32_t Hq,
                                                            int32_t D, void* out, int32_t out_kind,
                                                            float* lse) {
  const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // row * Hq + head
  const int64_t total = (int64_t)rows * Hq;
  if (rh >= total) return;
  auto logit = [&](int s) -> float { return part_lse[(int64_t)s * total + rh]; };
  merge_row<C, K_F32>(S, D, logit, part_o + rh * D, total * D, out, rh * D, out_kind, lse, rh);
}

template <int C, int PK>
__global__ __launch_bounds__(256) void segment_combine_kernel(
    const void* __restrict__ part_o, const float* __restrict__ part_lse,
    const int32_t* __restrict__ used, const float* __restrict__ bias, int32_t N, int32_t G,
    int32_t Hq, int32_t D, void* out, int32_t out_kind, float* lse) {
  const int64_t nh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // n * Hq + h
  if (nh >= (int64_t)N * Hq) return;
  const int64_t n = nh / Hq;
  const int h = (int)(nh - n * Hq);
  auto logit = [&](int g) -> float {
    if (used[n * G + g] <= 0) return kNegInf;
    const float prior = g < G - 1 ? bias[n * (G - 1) + g] : 0.f;
    return part_lse[(n * G + g) * Hq + h] + prior;
  };
  const int64_t eb = PK == K_F32 ? 4 : 2;
  const char* obase = static_cast<const char*>(part_o) + ((n * G) * Hq + h) * D * eb;
  merge_row<C, PK>(G, D, logit, obase, (int64_t)Hq * D, out, nh * D, out_kind, lse, nh);
}

__global__ void describe_kernel(const int32_t* __restrict__ table, int64_t bt_stride,
                                int32_t bt_width, const int32_t* __restrict__ seq_lens, int32_t B,
                                int32_t query_len, int32_t P, int32_t window, int32_t S,
                                int32_t chunk, int32_t* out_lens, int32_t* out_table,
                                int32_t out_width, int32_t* split_ranges) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const SeqView sv = seq_view(seq_lens[b], window, query_len, P, bt_width);
  out_lens[b] = sv.len;
  if (out_table)
    for (int j = 0; j < out_width; ++j)
      out_table[(int64_t)b * out_width + j] = table[(int64_t)b * bt_stride + table_column(sv, j, bt_width)];
  if (split_ranges)
    for (int s = 0; s < S; ++s) {
      const SplitRange r = split_range(sv, P, S, chunk, s);
      int32_t* o = split_ranges + ((int64_t)b * S + s) * 4;
      o[0] = r.first_page;
      o[1] = r.n_pages;
      o[2] = r.tok0;
      o[3] = r.n_tok;
    }
}

template <int C>
hipError_t launch_split_c(const float* part_o, const float* part_lse, int32_t S, int32_t rows,
                          int32_t Hq, int32_t D, void* out, int32_t out_kind, float* lse,
                          hipStream_t stream, int64_t grid) {
  hipLaunchKernelGGL(split_combine_kernel<C>, dim3((unsigned)grid), dim3(256), 0, stream, part_o,
                     part_lse, S, rows, Hq, D, out, out_kind, lse);
  return hipGetLastError();
}

template <int C, int PK>
hipError_t launch_segment_c(const void* part_o, const float* part_lse, const int32_t* used,
                            const float* bias, int32_t N, int32_t G, int32_t Hq, int32_t D,
                            void* out, int32_t out_kind, float* lse, hipStream_t stream,
                            int64_t grid) {
  hipLaunchKernelGGL((segment_combine_kernel<C, PK>), dim3((unsigned)grid), dim3(256), 0, stream,
                     part_o, part_lse, used, bias, N, G, Hq, D, out, out_kind, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_combine(const float* part_o, const float* part_lse, int32_t S,
                                int32_t rows, int32_t Hq, int32_t D, void* out, int32_t out_kind,
                                float* lse, hipStream_t stream) {
  const int64_t waves = (int64_t)rows * Hq;
  if (waves == 0) return hipSuccess;
  const int64_t grid = (waves + 3) / 4;
  if (D <= 64) return launch_split_c<1>(part_o, part_lse, S, rows, Hq, D, out, out_kind, lse, stream, grid);
  if (D <= 128) return launch_split_c<2>(part_o, part_lse, S, rows, Hq, D, out, out_kind, lse, stream, grid);
  return launch_split_c<4>(part_o, part_lse, S, rows, Hq, D, out, out_kind, lse, stream, grid);
}

hipError_t launch_segment_combine(const void* part_o, int32_t part_kind, const float* part_lse,
                                  const int32_t* used, const float* bias, int32_t N, int32_t G,
                                  int32_t Hq, int32_t D, void* out, int32_t out_kind, float* lse,
                                  hipStream_t stream) {
  const int64_t waves = (int64_t)N * Hq;
  if (waves == 0) return hipSuccess;
  const int64_t grid = (waves + 3) / 4;
#define PA_SEG(C)                                                                                \
  if (part_kind == K_F32)                                                                        \
    return launch_segment_c<C, K_F32>(part_o, part_lse, used, bias, N, G, Hq, D, out, out_kind, \
                                      lse, stream, grid);                                       \
  if (part_kind == K_BF16)                                                                       \
    return launch_segment_c<C, K_BF16>(part_o, part_lse, used, bias, N, G, Hq, D, out, out_kind,\
                                       lse, stream, grid);                                      \
  return launch_segment_c<C, K_FP16>(part_o, part_lse, used, bias, N, G, Hq, D, out, out_kind,  \
                                     lse, stream, grid);
  if (D <= 64) { PA_SEG(1) }
  if (D <= 128) { PA_SEG(2) }
  PA_SEG(4)
#undef PA_SEG
}

hipError_t launch_describe(const int32_t* block_table, int64_t bt_stride, int32_t bt_width,
                           const int32_t* seq_lens, int32_t B, int32_t query_len, int32_t P,
                           int32_t window, int32_t S, int32_t chunk, int32_t* out_lens,
                           int32_t* out_table, int32_t out_width, int32_t* split_ranges,
                           hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  const int threads = 64;
  const int grid = (B + threads - 1) / threads;
  hipLaunchKernelGGL(describe_kernel, dim3(grid), dim3(threads), 0, stream, block_table, bt_stride,
                     bt_width, seq_lens, B, query_len, P, window, S, chunk, out_lens, out_table,
                     out_width, split_ranges);
  return hipGetLastError();
}

}  // namespace pa
