// LSE-weighted combine kernels (Split-KV partials, DASH segments) and the
// device-side integer plan dump.
//
// Both combines are the merge that closes flash_dash_attention on the
// vllm.v1.attention.ops.dash_attention page: logits = partial LSE + prior,
// softmax over the live partials (dead ones excluded, all-dead giving zero
// weights), output = weighted sum of the live partial outputs.  Split-KV uses
// it with a zero prior and "live" meaning a finite partial LSE.
//
// One thread per V consecutive head-dim values of one (row, head).  Each
// thread reads the partial logits itself (the D/V threads of a row share them
// through the cache), so there is no cross-lane step, and it fetches the
// partial rows in batches of independent loads (8 Split-KV partials, 16 DASH
// segments), issued together with the logits and everything the logits need
// (segment lengths and biases are loaded unconditionally and selected
// afterwards, so a batch costs one round trip).  Batches are merged with a
// running maximum.  A dead partial's row and LSE (possibly never written)
// only ever meet a select, so they cannot leak into the result.

#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_plan.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kSplitBatch = 8;
constexpr int kSegmentBatch = 16;

// What the logit of one partial is formed from; settle() pins the loaded
// fields (an empty asm that reads them), so their loads are issued, and
// waited for, where the batch settles rather than inside a select's branch.
struct LseRaw {
  float lse;
  __device__ void settle() { asm volatile("" ::"v"(lse)); }
};
struct SegRaw {
  int used;
  float lse, bias;
  __device__ void settle() { asm volatile("" ::"v"(used), "v"(lse), "v"(bias)); }
};

template <int V, int PK>
__device__ __forceinline__ void load_vec(const void* base, int64_t i, float (&x)[V]) {
  if constexpr (PK == K_F32) {
    const float* p = reinterpret_cast<const float*>(base) + i;
    if constexpr (V == 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p);
      x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
    } else {
      x[0] = *p;
    }
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + i;
    uint16_t b[V];
    if constexpr (V == 4) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(p);
      b[0] = (uint16_t)w[0]; b[1] = (uint16_t)(w[0] >> 16);
      b[2] = (uint16_t)w[1]; b[3] = (uint16_t)(w[1] >> 16);
    } else {
      b[0] = *p;
    }
#pragma unroll
    for (int i2 = 0; i2 < V; ++i2)
      x[i2] = PK == K_BF16 ? __uint_as_float((uint32_t)b[i2] << 16) : (float)bitcast<_Float16>(b[i2]);
  }
}

template <int V>
__device__ __forceinline__ void store_vec(void* base, int64_t i, int kind, const float (&x)[V]) {
  if constexpr (V == 4) {
    store_row<4>(base, i, kind, x);
  } else if (kind == K_F32) {
    reinterpret_cast<float*>(base)[i] = x[0];
  } else if (kind == K_BF16) {
    reinterpret_cast<__bf16*>(base)[i] = (__bf16)x[0];
  } else {
    reinterpret_cast<_Float16*>(base)[i] = (_Float16)x[0];
  }
}

// Merge G partials of one (row, head) for this thread's V values.
// fetch(g) loads what the logit of partial g needs (a small struct with a
// settle() that pins its loaded fields), logit(raw, g) turns it into the
// natural-log logit (-inf: dead), load(g, x) fetches the partial's values.
// A batch issues every load first and settles them all before any logit is
// formed, so no load ends up behind a test of another (the compiler would
// otherwise move a load used on one side of a select into a branch, after a
// wait for the select's condition).  Returns the weighted mean in o and the
// merged LSE.
template <int V, int kBatch, typename FetchFn, typename LogitFn, typename LoadFn>
__device__ __forceinline__ float merge_partials(int G, FetchFn fetch, LogitFn logit, LoadFn load,
                                                float (&o)[V]) {
  float m = kNegInf, l = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) o[i] = 0.f;
  for (int g0 = 0; g0 < G; g0 += kBatch) {
    decltype(fetch(0)) raw[kBatch];
    float lg[kBatch], x[kBatch][V];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int g = g0 + u < G ? g0 + u : g0;  // past the end: a valid index, weight forced to 0
      raw[u] = fetch(g);
      load(g, x[u]);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) raw[u].settle();
#pragma unroll
    for (int u = 0; u < kBatch; ++u) lg[u] = g0 + u < G ? logit(raw[u], g0 + u) : kNegInf;
    float mb = m;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) mb = fmaxf(mb, lg[u]);
    if (mb == kNegInf) continue;  // every partial so far is dead
    if (mb > m) {
      const float a = fast_exp2((m - mb) * kLog2e);  // 0 while m is still -inf
      l *= a;
#pragma unroll
      for (int i = 0; i < V; ++i) o[i] *= a;
      m = mb;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = lg[u] == kNegInf ? 0.f : fast_exp2((lg[u] - m) * kLog2e);
      l += w;
#pragma unroll
      for (int i = 0; i < V; ++i) o[i] = w > 0.f ? o[i] + w * x[u][i] : o[i];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) o[i] *= inv;
  return l > 0.f ? m + logf(l) : kNegInf;
}

template <int V>
__global__ __launch_bounds__(256) void split_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_lse,
                                                            int32_t S, int32_t rows, int32_t Hq,
                                                            int32_t D, void* out, int32_t out_kind,
                                                            float* lse) {
  const int64_t total = (int64_t)rows * Hq;
  const int tpr = D / V;  // threads per (row, head)
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rh = t / tpr;  // row * Hq + head
  if (rh >= total) return;
  const int d0 = (int)(t - rh * tpr) * V;
  auto fetch = [&](int s) { return LseRaw{part_lse[(int64_t)s * total + rh]}; };
  auto logit = [](const LseRaw& r, int) { return r.lse; };
  auto load = [&](int s, float (&x)[V]) {
    load_vec<V, K_F32>(part_o, ((int64_t)s * total + rh) * D + d0, x);
  };
  float o[V];
  const float L = merge_partials<V, kSplitBatch>(S, fetch, logit, load, o);
  store_vec<V>(out, rh * D + d0, out_kind, o);
  if (lse && d0 == 0) lse[rh] = L;
}

template <int V, int PK>
__global__ __launch_bounds__(256) void segment_combine_kernel(
    const void* __restrict__ part_o, const float* __restrict__ part_lse,
    const int32_t* __restrict__ used, const float* __restrict__ bias, int32_t N, int32_t G,
    int32_t Hq, int32_t D, void* out, int32_t out_kind, float* lse) {
  const int tpr = D / V;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nh = t / tpr;  // n * Hq + h
  if (nh >= (int64_t)N * Hq) return;
  const int d0 = (int)(t - nh * tpr) * V;
  const int64_t n = nh / Hq;
  const int h = (int)(nh - n * Hq);
  // Without remote segments there is no bias row (the pointer may be NULL):
  // the bias load then rereads the LSE row and is dropped, as it is for the
  // local segment (g = G - 1), which rereads the last remote bias.
  const float* brow = G > 1 ? bias + n * (G - 1) : part_lse;
  auto fetch = [&](int g) {
    return SegRaw{used[n * G + g], part_lse[(n * G + g) * Hq + h], brow[g < G - 1 ? g : (G > 1 ? G - 2 : 0)]};
  };
  auto logit = [&](const SegRaw& r, int g) {
    return r.used <= 0 ? kNegInf : r.lse + (g < G - 1 ? r.bias : 0.f);
  };
  auto load = [&](int g, float (&x)[V]) {
    load_vec<V, PK>(part_o, ((n * G + g) * Hq + h) * D + d0, x);
  };
  float o[V];
  const float L = merge_partials<V, kSegmentBatch>(G, fetch, logit, load, o);
  store_vec<V>(out, nh * D + d0, out_kind, o);
  if (lse && d0 == 0) lse[nh] = L;
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

template <int V>
hipError_t launch_split_v(const float* part_o, const float* part_lse, int32_t S, int32_t rows,
                          int32_t Hq, int32_t D, void* out, int32_t out_kind, float* lse,
                          hipStream_t stream) {
  const int64_t threads = (int64_t)rows * Hq * (D / V);
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(split_combine_kernel<V>, dim3((unsigned)grid), dim3(256), 0, stream, part_o,
                     part_lse, S, rows, Hq, D, out, out_kind, lse);
  return hipGetLastError();
}

template <int V, int PK>
hipError_t launch_segment_v(const void* part_o, const float* part_lse, const int32_t* used,
                            const float* bias, int32_t N, int32_t G, int32_t Hq, int32_t D,
                            void* out, int32_t out_kind, float* lse, hipStream_t stream) {
  const int64_t threads = (int64_t)N * Hq * (D / V);
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((segment_combine_kernel<V, PK>), dim3((unsigned)grid), dim3(256), 0, stream,
                     part_o, part_lse, used, bias, N, G, Hq, D, out, out_kind, lse);
  return hipGetLastError();
}

// Four values per thread when the rows allow whole-vector accesses.
bool vec4_ok(const void* in, int in_bytes, const void* out, int out_bytes, int D) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(in), b = reinterpret_cast<uintptr_t>(out);
  return D % 4 == 0 && a % (4 * in_bytes) == 0 && b % (4 * out_bytes) == 0;
}

int elem_bytes(int kind) { return kind == K_F32 ? 4 : 2; }

}  // namespace

hipError_t launch_split_combine(const float* part_o, const float* part_lse, int32_t S,
                                int32_t rows, int32_t Hq, int32_t D, void* out, int32_t out_kind,
                                float* lse, hipStream_t stream) {
  if ((int64_t)rows * Hq == 0) return hipSuccess;
  if (vec4_ok(part_o, 4, out, elem_bytes(out_kind), D))
    return launch_split_v<4>(part_o, part_lse, S, rows, Hq, D, out, out_kind, lse, stream);
  return launch_split_v<1>(part_o, part_lse, S, rows, Hq, D, out, out_kind, lse, stream);
}

hipError_t launch_segment_combine(const void* part_o, int32_t part_kind, const float* part_lse,
                                  const int32_t* used, const float* bias, int32_t N, int32_t G,
                                  int32_t Hq, int32_t D, void* out, int32_t out_kind, float* lse,
                                  hipStream_t stream) {
  if ((int64_t)N * Hq == 0) return hipSuccess;
  const bool v4 = vec4_ok(part_o, elem_bytes(part_kind), out, elem_bytes(out_kind), D);
#define PA_SEG(V)                                                                                 \
  if (part_kind == K_F32)                                                                         \
    return launch_segment_v<V, K_F32>(part_o, part_lse, used, bias, N, G, Hq, D, out, out_kind, \
                                      lse, stream);                                              \
  if (part_kind == K_BF16)                                                                        \
    return launch_segment_v<V, K_BF16>(part_o, part_lse, used, bias, N, G, Hq, D, out, out_kind,\
                                       lse, stream);                                             \
  return launch_segment_v<V, K_FP16>(part_o, part_lse, used, bias, N, G, Hq, D, out, out_kind,  \
                                     lse, stream);
  if (v4) { PA_SEG(4) }
  PA_SEG(1)
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
