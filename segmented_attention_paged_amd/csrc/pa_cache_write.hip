// Paged K/V cache write (page vllm.v1.attention.backends.flashinfer_ts,
// do_kv_cache_update): the key and value rows of each new token go to slot
// s % P of page s // P, s = slot_mapping[token], K into the first D values of
// the slot's row and V into the last D (or into separate K and V planes: any
// strides).  Padding slots (negative) and slots past the pool write nothing.
// A cache of the input's own type receives the input bits; an e4m3fn cache
// receives e4m3fn(x / scale), the quotient rounded to fp32 and then to the
// nearest finite e4m3fn value (ties to even, saturating at +-448, NaN kept),
// so that scale * stored is what the attention kernels read back.
//
// The kernel is a pure HBM scatter of pieces of one (token, kv head) row: 8
// values per thread for a 16-bit cache (16 bytes in, 16 out), 16 for an fp8
// cache when D is a multiple of 16 (32 bytes in, 16 out), else 8 (16 in, 8 out).

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

// e4m3fn codes of two fp32 values (low byte: a, next byte: b): nearest finite
// value, ties to the even code, |x| >= 448 and +-inf saturating to +-448, NaN
// -> 0x7F with the input's sign.  v_cvt_pk_fp8_f32 (OCP e4m3fn on gfx950)
// rounds to nearest even and was checked bit for bit against a software
// encoder on every bf16 value and 2M further fp32 values below 448 in
// magnitude; above that it returns NaN, so magnitudes >= 448 are clamped to
// 448 first, and its NaN code (always 0xFF) gets the input's sign back.
__device__ __forceinline__ uint32_t e4m3fn_pair(float a, float b) {
  auto saturate = [](uint32_t u) {
    const uint32_t m = u & 0x7FFFFFFFu;
    return (m >= 0x43E00000u && m <= 0x7F800000u) ? ((u & 0x80000000u) | 0x43E00000u) : u;
  };
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(saturate(ua)),
                                                        __uint_as_float(saturate(ub)), 0, false) &
               0xFFFFu;
  const uint32_t nan_a = ((ua >> 24) & 0x80u) | 0x7Fu, nan_b = ((ub >> 24) & 0x80u) | 0x7Fu;
  r = (ua & 0x7FFFFFFFu) > 0x7F800000u ? (r & 0xFF00u) | nan_a : r;
  r = (ub & 0x7FFFFFFFu) > 0x7F800000u ? (r & 0x00FFu) | (nan_b << 8) : r;
  return r;
}

template <int IN>
__device__ __forceinline__ float to_f32(uint32_t half_bits) {
  if constexpr (IN == K_BF16) return __uint_as_float(half_bits << 16);
  return (float)bitcast<_Float16>((uint16_t)half_bits);
}

// One thread moves VPT consecutive values of one (token, kv head) row: VPT = 8
// (a 16-byte load and store) for a 16-bit cache, 16 for an fp8 cache (two
// 16-byte loads, one 16-byte store).  WIDE: 64-bit thread and slot arithmetic
// (more than 2^31 threads or slots); otherwise 32-bit divisions.
template <int IN, bool FP8, bool WIDE, int VPT>
__global__ __launch_bounds__(256) void kv_write_kernel(KVWriteParams p) {
  static_assert(VPT == 8 || (FP8 && VPT == 16), "values per thread");
  const int tpr = 2 * p.D / VPT;  // threads per (token, head)
  int64_t tok, page, off;
  int e, h;
  if constexpr (WIDE) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = t / tpr;  // token * Hkv + head
    if (row >= (int64_t)p.T * p.Hkv) return;
    e = (int)(t - row * tpr) * VPT;
    tok = row / p.Hkv;
    h = (int)(row - tok * p.Hkv);
  } else {
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    const uint32_t r32 = t / (uint32_t)tpr;
    if (r32 >= (uint32_t)p.T * (uint32_t)p.Hkv) return;
    e = (int)(t - r32 * (uint32_t)tpr) * VPT;
    const uint32_t t32 = r32 / (uint32_t)p.Hkv;
    tok = t32;
    h = (int)(r32 - t32 * (uint32_t)p.Hkv);
  }
  // e: value index in [K | V], 0 .. 2D-1
  const int64_t slot = p.slot_mapping[tok];
  if (slot < 0 || slot >= p.capacity) return;
  if constexpr (WIDE) {
    page = slot / p.P;
    off = slot - page * p.P;
  } else {
    const uint32_t s32 = (uint32_t)slot, pg = s32 / (uint32_t)p.P;
    page = pg;
    off = s32 - pg * (uint32_t)p.P;
  }
  const bool is_v = e >= p.D;
  const int d = is_v ? e - p.D : e;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(is_v ? p.value : p.key) +
                        tok * (is_v ? p.value_stride : p.key_stride) + (int64_t)h * p.D + d;
  u32x4 x[VPT / 8];
#pragma unroll
  for (int c = 0; c < VPT / 8; ++c) x[c] = *reinterpret_cast<const u32x4*>(src + 8 * c);
  const int64_t dst_off = page * p.page_stride + (int64_t)h * p.head_stride + off * p.token_stride + d;
  if constexpr (!FP8) {
    char* dst = static_cast<char*>(is_v ? p.v_cache : p.k_cache) + dst_off * 2;
    *reinterpret_cast<u32x4*>(dst) = x[0];
  } else {
    // x / scale rounded to fp32, computed as fp32(double(x) * RN64(1 / scale)).
    // This is the correctly rounded fp32 quotient: the product is within 2^-52
    // (relative) of x / scale, while the quotient of two 24-bit numbers is
    // never a float rounding midpoint and never nearer than ~2^-50 to one
    // (only quotients in the fp32 subnormal range escape the argument, and
    // they all encode to +-0 in e4m3fn either way).
    const double inv = is_v ? p.v_inv : p.k_inv;
    uint32_t w[VPT / 4];
#pragma unroll
    for (int i = 0; i < VPT / 2; ++i) {  // values 2i, 2i+1 = the two halves of dword i
      const uint32_t dw = x[i >> 2][i & 3];
      const float q0 = (float)((double)to_f32<IN>(dw & 0xFFFFu) * inv);
      const float q1 = (float)((double)to_f32<IN>(dw >> 16) * inv);
      const uint32_t pair = e4m3fn_pair(q0, q1);
      if (i & 1) w[i >> 1] |= pair << 16;
      else w[i >> 1] = pair;
    }
    char* dst = static_cast<char*>(is_v ? p.v_cache : p.k_cache) + dst_off;
    if constexpr (VPT == 16) *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    else *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
  }
}

template <int IN, bool FP8, int VPT>
hipError_t launch_kv_write_t(const KVWriteParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.T * p.Hkv * (2 * p.D / VPT);
  if (threads == 0) return hipSuccess;
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.capacity > 0x7fffffffLL || grid * 256 > 0x7fffffffLL)
    hipLaunchKernelGGL((kv_write_kernel<IN, FP8, true, VPT>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((kv_write_kernel<IN, FP8, false, VPT>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_write(const KVWriteParams& p, int in_kind, int cache_kind, hipStream_t stream) {
  const bool fp8 = cache_kind == K_FP8;
  const bool wide16 = fp8 && p.D % 16 == 0;  // fp8 rows in 16-value pieces
  if (in_kind == K_BF16) {
    if (!fp8) return launch_kv_write_t<K_BF16, false, 8>(p, stream);
    return wide16 ? launch_kv_write_t<K_BF16, true, 16>(p, stream) : launch_kv_write_t<K_BF16, true, 8>(p, stream);
  }
  if (!fp8) return launch_kv_write_t<K_FP16, false, 8>(p, stream);
  return wide16 ? launch_kv_write_t<K_FP16, true, 16>(p, stream) : launch_kv_write_t<K_FP16, true, 8>(p, stream);
}

}  // namespace pa
