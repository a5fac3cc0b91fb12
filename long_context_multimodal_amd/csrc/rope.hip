// Rotary position embedding at global token positions (gfx950).
//
// "LongVILA Guide: 2M Context Multi-Modal AI Model", section "Three-Stage
// Long-Context Alignment Curriculum", stage 2: the base theta of the rotary
// embedding is raised to 10,000,000 for the long-context stages.  Half-split
// pairs: (x[i], x[i+d/2]) of a token at position p turns by the angle
// p * theta^(-2i/d); the inverse turns by minus that angle (it maps gradients
// with respect to rotated queries/keys back to the unrotated ones).
//
// One pass over the tensor, HBM-bound: one thread per (token, 8 consecutive
// pairs), looping over heads, so the 8 angles -- computed in fp64 from the
// exact integer position, which at positions up to 2^21 an fp32 product
// would get wrong by up to a tenth of a radian -- are shared by all heads.
// bf16 results are rounded fp64 -> fp32 -> bf16 (nearest even), fp32 results
// fp64 -> fp32.  In place (y == x) is allowed: each thread reads its two
// 8-element pieces before writing them.
#include "common.h"
#include "kernels.h"

namespace mmsp {
namespace {

template <int D, bool BF16>
__global__ void __launch_bounds__(256) rope_kernel(const void* __restrict__ x, void* y,
                                                   const int32_t* __restrict__ pos, int s, int h,
                                                   double theta, int inverse) {
  constexpr int HALF = D / 2;
  constexpr int GROUPS = HALF / 8;  // 8 pairs per thread
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= s * GROUPS) return;
  const int tok = t / GROUPS;
  const int i0 = (t % GROUPS) * 8;
  const double p = (double)pos[tok];
  double cs[8], sn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double inv_freq = pow(theta, -2.0 * (double)(i0 + e) / (double)D);
    sincos(p * inv_freq, &sn[e], &cs[e]);
    if (inverse) sn[e] = -sn[e];
  }
  for (int hd = 0; hd < h; ++hd) {
    const size_t base = ((size_t)tok * h + hd) * D + i0;
    double a[8], b[8];
    if constexpr (BF16) {
      const u32x4 va = *(const u32x4*)((const uint16_t*)x + base);
      const u32x4 vb = *(const u32x4*)((const uint16_t*)x + base + HALF);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        a[2 * w] = bf16_lo(va[w]);
        a[2 * w + 1] = bf16_hi(va[w]);
        b[2 * w] = bf16_lo(vb[w]);
        b[2 * w + 1] = bf16_hi(vb[w]);
      }
    } else {
      const f32x4* pa = (const f32x4*)((const float*)x + base);
      const f32x4* pb = (const f32x4*)((const float*)x + base + HALF);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const f32x4 ua = pa[w], ub = pb[w];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[4 * w + e] = ua[e];
          b[4 * w + e] = ub[e];
        }
      }
    }
    float ra[8], rb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ra[e] = (float)(a[e] * cs[e] - b[e] * sn[e]);
      rb[e] = (float)(b[e] * cs[e] + a[e] * sn[e]);
    }
    if constexpr (BF16) {
      u32x4 oa, ob;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        oa[w] = pack_bf16x2(ra[2 * w], ra[2 * w + 1]);
        ob[w] = pack_bf16x2(rb[2 * w], rb[2 * w + 1]);
      }
      *(u32x4*)((uint16_t*)y + base) = oa;
      *(u32x4*)((uint16_t*)y + base + HALF) = ob;
    } else {
      f32x4* qa = (f32x4*)((float*)y + base);
      f32x4* qb = (f32x4*)((float*)y + base + HALF);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        qa[w] = f32x4{ra[4 * w], ra[4 * w + 1], ra[4 * w + 2], ra[4 * w + 3]};
        qb[w] = f32x4{rb[4 * w], rb[4 * w + 1], rb[4 * w + 2], rb[4 * w + 3]};
      }
    }
  }
}

template <int D>
hipError_t launch_rope_d(const void* x, void* y, bool bf16, const int32_t* pos, int s, int h,
                         double theta, int inverse, hipStream_t stream) {
  const int threads = s * (D / 16);
  const dim3 grid((threads + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL((rope_kernel<D, true>), grid, dim3(256), 0, stream, x, y, pos, s, h, theta,
                       inverse);
  else
    hipLaunchKernelGGL((rope_kernel<D, false>), grid, dim3(256), 0, stream, x, y, pos, s, h,
                       theta, inverse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const void* x, void* y, bool bf16, const int32_t* pos, int s, int h, int d,
                       double theta, int inverse, hipStream_t stream) {
  return d == 64 ? launch_rope_d<64>(x, y, bf16, pos, s, h, theta, inverse, stream)
                 : launch_rope_d<128>(x, y, bf16, pos, s, h, theta, inverse, stream);
}

}  // namespace mmsp
