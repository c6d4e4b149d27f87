// Device-side helpers shared by the WBMM kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wbmm {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;  // 4 waves of 64 lanes per workgroup

// ---------------------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even; NaN stays NaN (quietened).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p, size_t i);
template <> __device__ __forceinline__ float load_f32<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t* p, size_t i) {
  return bf2f(p[i]);
}

// ---------------------------------------------------------------------------- fast division
// Division by a runtime divisor d >= 1 through a 64-bit reciprocal m = ceil(2^64 / d): for any
// 32-bit a the error of a*m/2^64 against a/d is below 2^-32 while a/d's fractional part is at
// most 1 - 1/d, so the high half of the product is floor(a/d) exactly.
struct FastDiv {
  uint32_t d;
  uint32_t pad_;
  uint64_t m;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t a, FastDiv f) {
  return f.d == 1 ? a : (uint32_t)__umul64hi((uint64_t)a, f.m);
}
__device__ __forceinline__ void fdivmod(uint32_t a, FastDiv f, uint32_t& q, uint32_t& r) {
  q = fdiv(a, f);
  r = a - q * f.d;
}

// ---------------------------------------------------------------------------- map addressing
// Offset of element (b, c, h, v) in a dense map of shape (B, C, H, W) stored NCHW (layout 0) or
// NHWC (layout 1).
__device__ __forceinline__ size_t map_off(int layout, int b, int c, int h, int v, int C, int H,
                                          int W) {
  return layout == 0 ? (((size_t)b * C + c) * H + h) * W + v
                     : (((size_t)b * H + h) * W + v) * C + c;
}

__device__ __forceinline__ v4f mfma_f32(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_bf16(u32x4 a, u32x4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                 __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------- wave sums
// x of lane (i - n) within the lane's row of 16 (ROW_SHR), or of the broadcast source lane; 0
// where there is none or the row is masked off. Both 32-bit halves move the same way.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xf, true);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// Sum of x over the 64 lanes of a wave, in a fixed order, left in lane 63: within each row of 16
// lanes, shifted copies are added (row_shr 1, 2, 4, 8: lane 15 then holds its row's sum); the sum
// of row 0 is added into row 1 and that of row 2 into row 3 (row_bcast 15), then lane 31's into
// rows 2 and 3 (row_bcast 31). VALU moves only (no LDS traffic, unlike lane shuffles).
__device__ __forceinline__ double wave_sum_f64_last(double x) {
  x += dpp_f64<0x111, 0xf>(x);
  x += dpp_f64<0x112, 0xf>(x);
  x += dpp_f64<0x114, 0xf>(x);
  x += dpp_f64<0x118, 0xf>(x);
  x += dpp_f64<0x142, 0xa>(x);
  x += dpp_f64<0x143, 0xc>(x);
  return x;
}

}  // namespace wbmm
