// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Global positions of a local tensor's rows: up to two runs, stored in order.
// Row i < len0 sits at start0 + i, otherwise at start1 + (i - len0).
struct DevSegs {
  int32_t start0;
  int32_t start1;
  int32_t len0;  // rows in the first run (the total when there is one run)
  int32_t len;   // total rows
};

__device__ __forceinline__ int32_t seg_pos(const DevSegs& s, int32_t row) {
  return row < s.len0 ? s.start0 + row : s.start1 + (row - s.len0);
}

// Smallest and largest global position of rows [r0, r1) (r0 < r1 <= len).
__device__ __forceinline__ void seg_range(const DevSegs& s, int32_t r0, int32_t r1,
                                          int32_t& lo, int32_t& hi) {
  lo = INT32_MAX;
  hi = INT32_MIN;
  if (r0 < s.len0) {
    int32_t e = r1 < s.len0 ? r1 : s.len0;
    lo = s.start0 + r0;
    hi = s.start0 + e - 1;
  }
  if (r1 > s.len0) {
    int32_t b = r0 > s.len0 ? r0 : s.len0;
    int32_t a = s.start1 + (b - s.len0), z = s.start1 + (r1 - 1 - s.len0);
    lo = a < lo ? a : lo;
    hi = z > hi ? z : hi;
  }
}

// bf16 <-> fp32 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }
__device__ __forceinline__ float from_bf16(bf16 x) { return (float)x; }

// Maxima of values that are never NaN (scores of finite inputs, or -inf):
// single v_max / v_max3 instructions. fmaxf would first quiet possible
// signalling NaNs of every operand, doubling the instruction count.
__device__ __forceinline__ float max2_nn(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_nn(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Value of `x` held by lane (lane ^ 32), via the gfx950 32-lane swap.
__device__ __forceinline__ float partner32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float partner32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace ra
