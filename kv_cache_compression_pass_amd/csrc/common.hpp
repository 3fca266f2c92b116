// Device helpers shared by the libkvc kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 32x32x16 bf16 matrix-core product, fp32 accumulate.
// Lane l supplies A[m = l%32][k = 8*(l/32) + j] and B[k = 8*(l/32) + j][n = l%32], j = 0..7, and
// holds D[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32] in element i (i = 0..15).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row (m) index of accumulator element i held by a lane in half `hi` (= lane / 32).
__device__ __forceinline__ int acc_row(int i, int hi) { return 8 * (i >> 2) + 4 * hi + (i & 3); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exchange with the lane 32 apart (the other half of a 32x32 accumulator column).
__device__ __forceinline__ float swap_half(float x) { return __shfl_xor(x, 32, 64); }

// max of three values with one v_max3_f32.  fmaxf() on matrix-core results makes the compiler
// quiet possible signalling NaNs first (an extra instruction per operand); the values here are
// never NaN, so the raw instruction gives the same result.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// max / sum of a value and the one held 32 lanes away, on the VALU (v_permlane32_swap): lane
// l < 32 sees (x[l], x[l + 32]), lane l >= 32 sees (x[l - 32], x[l]); both get the same result.
// (max: values are never NaN here, see max3_raw.)
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Record a device-side data error in the workspace status word.
__device__ __forceinline__ void set_status(int32_t* status, int32_t code) {
  if (status) atomicOr(status, code);
}

__device__ __forceinline__ bool valid_width(uint32_t b) {
  return b == 0 || b == 2 || b == 4 || b == 8 || b == 16;
}

// Exclusive prefix sum of one uint64 per thread over a block of NT threads (NT % 64 == 0);
// *total receives the block total.  sh holds NT / 64 entries.  Every thread must call it.
template <int NT>
__device__ __forceinline__ uint64_t block_excl_scan(uint64_t v, uint64_t* total, uint64_t* sh) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = __shfl_up((uint32_t)x, o, 64), hi = __shfl_up((uint32_t)(x >> 32), o, 64);
    if (lane >= o) x += ((uint64_t)hi << 32) | lo;
  }
  if (lane == 63) sh[wid] = x;
  __syncthreads();
  if (wid == 0) {
    uint64_t y = lane < NW ? sh[lane] : 0;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      const uint32_t lo = __shfl_up((uint32_t)y, o, 64), hi = __shfl_up((uint32_t)(y >> 32), o, 64);
      if (lane >= o) y += ((uint64_t)hi << 32) | lo;
    }
    if (lane < NW) sh[lane] = y;       // inclusive wave totals
  }
  __syncthreads();
  const uint64_t r = (wid > 0 ? sh[wid - 1] : 0) + x - v;
  *total = sh[NW - 1];
  __syncthreads();                     // sh may be reused by the caller's next scan
  return r;
}

}  // namespace kvc
