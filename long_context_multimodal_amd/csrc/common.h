// Device helpers shared by the gfx950 kernels of libmmsp.so.
//
// Matrix-core conventions (CDNA4 v_mfma_f32_32x32x16_bf16, 64-lane wave):
//   A (32 x 16, M x K): lane l supplies row m = l % 32, k = 8*(l/32) + 0..7
//   B (16 x 32, K x N): lane l supplies col n = l % 32, k = 8*(l/32) + 0..7
//   C (32 x 32, fp32) : lane l holds col n = l % 32 and, for i = 0..15,
//                       row m = 8*(i/4) + 4*(l/32) + (i%4)
// Hence an accumulator row index r of lane-half hh = l/32 takes the values
// {0,1,2,3, 8,9,10,11, 16..19, 24..27} (+4 for hh = 1).  When a C tile is fed
// back as the B operand of the next contraction (K = its row index), the
// first 8 accumulator entries form K-step 0 and the last 8 K-step 1, with
// the row set of each lane-half acting as that half's k = 0..7.  The operand
// paired with it must list its rows in the same order; kPerm16 below gives
// the position of row r (0..15 within a K-step) in that order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmsp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position, within one K-step of 16 rows, at which row r is stored so that
// lane-half 0 reads rows {0-3, 8-11} and lane-half 1 rows {4-7, 12-15} as 8
// consecutive elements: quads 1 and 2 trade places.
__device__ __forceinline__ constexpr int kPerm16(int r) {
  const int quad = r >> 2;
  const int q2 = (quad == 1) ? 2 : (quad == 2 ? 1 : quad);
  return (q2 << 2) | (r & 3);
}

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// max / sum of a value with the same lane in the other half of the wave
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup order that keeps consecutive logical tiles on one XCD: the
// dispatcher deals workgroup b to XCD b % 8, so logical tile
// (b % 8) * (n / 8) + b / 8 runs on XCD b % 8 and each XCD sweeps one
// contiguous range of logical tiles (sharing its L2).
__device__ __forceinline__ int xcd_logical_block(int b, int n) {
  if ((n & 7) != 0) return b;
  return (b & 7) * (n >> 3) + (b >> 3);
}

}  // namespace mmsp
