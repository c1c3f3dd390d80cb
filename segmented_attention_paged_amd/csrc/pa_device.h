// Device-side building blocks for gfx950 (CDNA4): MFMA wrappers, 16-bit
// packing, fp8 decoding and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int v2i32 __attribute__((ext_vector_type(2)));

// Element kinds (numerically equal to the public pa_dtype codes).
enum Kind : int { K_BF16 = 1, K_FP16 = 2, K_FP8 = 3, K_F32 = 4 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size");
  return __builtin_bit_cast(To, f);
}

// S^T tile: 16 keys x 16 rows, contraction over 32 head-dim values.
// A = K (lane l: key l%16, 8 values at k = 8*(l/16)..), B = Q^T (lane l:
// row l%16, same k), C: lane l holds keys 4*(l/16)+i, row l%16.
template <int T>
__device__ __forceinline__ f32x4 mfma_16x16x32(const u32x4& a, const u32x4& b, f32x4 c) {
  if constexpr (T == K_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8>(a), bitcast<f16x8>(b), c, 0, 0, 0);
}

// Operand types of a query kind: the S^T operands (K and Q^T, 32 head-dim
// values per lane group) and the element type of P and V in O^T += V^T P^T.
// A 16-bit query runs both products in its own type; an fp8 query runs S^T
// on fp8 MFMA (the cache is fp8 too) and O^T in bf16.
template <int QT>
struct QTypes {
  using QOp = u32x4;  // 8 16-bit values
  static constexpr int PV = QT;
};
template <>
struct QTypes<K_FP8> {
  using QOp = u32x2;  // 8 e4m3fn bytes
  static constexpr int PV = K_BF16;
};

// S^T tile for a query kind (the mfma_16x16x32 layout above for every kind;
// gfx950's fp8 MFMA takes OCP e4m3fn, checked on the GPU by a probe).
template <int QT>
__device__ __forceinline__ f32x4 qk_mfma(const typename QTypes<QT>::QOp& a,
                                         const typename QTypes<QT>::QOp& b, f32x4 c) {
  if constexpr (QT == K_FP8)
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(bitcast<long>(a), bitcast<long>(b), c, 0, 0, 0);
  else
    return mfma_16x16x32<QT>(a, b, c);
}

// O^T tile: 16 head-dim values x 16 rows, contraction over 16 keys.
// A = V^T (lane l: dim-row l%16, keys 4*(l/16)+i), B = P^T (lane l: keys
// 4*(l/16)+i, row l%16) -- exactly the C layout of mfma_16x16x32 above.
template <int T>
__device__ __forceinline__ f32x4 mfma_16x16x16(const u32x2& a, const u32x2& b, f32x4 c) {
  if constexpr (T == K_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bitcast<i16x4>(a), bitcast<i16x4>(b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(bitcast<f16x4>(a), bitcast<f16x4>(b), c, 0, 0, 0);
}

// Two floats -> one dword of two 16-bit values (round to nearest even), lo first.
template <int T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (T == K_BF16) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return bitcast<uint32_t>(r);
  } else {
    f16x2 r = {(_Float16)lo, (_Float16)hi};
    return bitcast<uint32_t>(r);
  }
}

// Four e4m3fn bytes -> two dwords of 16-bit values (bytes 0,1 then 2,3),
// exact: every e4m3fn value is representable in bf16 and in fp16.
template <int T>
__device__ __forceinline__ void fp8x4_to_16(uint32_t x, uint32_t& lo, uint32_t& hi) {
  if constexpr (T == K_BF16) {
    lo = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
    hi = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
  } else {
    lo = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
    hi = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true));
  }
}

// 16-bit halves: keys (a, b) of one head-dim position -> one MFMA dword.
__device__ __forceinline__ uint32_t lo_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// max of two floats as gfx950's v_maximum_f32 (NaN-propagating): no quieting of
// the operands first, which fmaxf needs in IEEE mode.  The attention logits it
// sees are finite or -inf.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Reductions across the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48).
// gfx950 lane swaps: permlane32_swap(a, b) exchanges lanes 32..63 of a with
// lanes 0..31 of b; permlane16_swap(a, b) exchanges the odd 16-lane rows of a
// with the even rows of b.  Called with a == b == x, element-wise op of the
// two results is op(x[l], x[l ^ 32]) (resp. x[l ^ 16]) in every lane.
__device__ __forceinline__ float xor32_pair(float x, bool max_op) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return max_op ? vmax(a, b) : a + b;
}
__device__ __forceinline__ float xor16_pair(float x, bool max_op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return max_op ? vmax(a, b) : a + b;
}
__device__ __forceinline__ float max_across_groups(float x) { return xor32_pair(xor16_pair(x, true), true); }
__device__ __forceinline__ float sum_across_groups(float x) { return xor32_pair(xor16_pair(x, false), false); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding: vmcnt[3:0] in bits 3:0 and
// vmcnt[5:4] in bits 15:14; expcnt = 7 and lgkmcnt = 15 mean "do not wait").
constexpr int vmcnt_imm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 0x3) << 14); }
// s_waitcnt immediate that waits for every LDS / scalar-memory operation of this
// wave (lgkmcnt = 0) and for nothing else.
constexpr int kLgkmcnt0 = 0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);

// Store `n` consecutive floats (n = 4 or 8) converted to the output kind.
template <int N>
__device__ __forceinline__ void store_row(void* base, int64_t elem_off, int kind, const float* v) {
  if (kind == K_F32) {
    float* o = reinterpret_cast<float*>(base) + elem_off;
#pragma unroll
    for (int i = 0; i < N; i += 4) *reinterpret_cast<f32x4*>(o + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
  } else {
    uint16_t* o = reinterpret_cast<uint16_t*>(base) + elem_off;
    uint32_t w[N / 2];
    if (kind == K_BF16) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) w[i] = pack2<K_BF16>(v[2 * i], v[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) w[i] = pack2<K_FP16>(v[2 * i], v[2 * i + 1]);
    }
    if constexpr (N == 8) {
      *reinterpret_cast<u32x4*>(o) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      *reinterpret_cast<u32x2*>(o) = u32x2{w[0], w[1]};
    }
  }
}

}  // namespace pa
