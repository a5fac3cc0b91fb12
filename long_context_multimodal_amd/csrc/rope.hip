// Rotary position embedding at global token positions (gfx950).
//
// "LongVILA Guide: 2M Context Multi-Modal AI Model", section "Three-Stage
// Long-Context Alignment Curriculum", stage 2: the base theta of the rotary
// embedding is raised to 10,000,000 for the long-context stages.  Half-split
// pairs: (x[i], x[i+d/2]) of a token at position p turns by the angle
// p * theta^(-2i/d); the inverse turns by minus that angle (it maps gradients
// with respect to rotated queries/keys back to the unrotated ones).
//
// One pass over the tensor, HBM-bound.  A block takes `tpb` consecutive tokens:
// its threads first compute the tokens' angles once each -- in fp64 from the
// exact integer position, since at positions up to 2^21 an fp32 product would
// be off by up to a tenth of a radian -- into LDS, then stream over the
// (token, head, 8 consecutive pairs) units of those tokens, four per thread
// with every load issued before the first store, so enough 16-byte loads are
// in flight to cover HBM latency at any head count.  bf16 results are
// rounded fp64 -> fp32 -> bf16 (nearest even), fp32 results fp64 -> fp32.
// In place (y == x) is allowed: each unit's two 8-element pieces are read
// before they are written, and no two units share an element.
#include "common.h"
#include "kernels.h"

namespace mmsp {
namespace {

constexpr int ROPE_THREADS = 256;
constexpr int ROPE_UNROLL = 4;
// largest LDS angle table: tpb * D/2 entries of (cos, sin) in fp64, 32 KiB
constexpr int ROPE_MAX_ANGLES = 2048;

template <bool BF16>
struct Piece;  // 8 consecutive elements of one half of a head row
template <>
struct Piece<true> {
  u32x4 v;
};
template <>
struct Piece<false> {
  f32x4 v[2];
};

template <int D, bool BF16>
__global__ void __launch_bounds__(ROPE_THREADS)
    rope_kernel(const void* __restrict__ x, void* y, const int32_t* __restrict__ pos, int s, int h,
                int tpb, double theta, int inverse) {
  constexpr int HALF = D / 2;
  constexpr int GROUPS = HALF / 8;  // 8 pairs per unit
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  extern __shared__ double s_tab[];  // cos then sin, tpb * HALF each
  double* s_cos = s_tab;
  double* s_sin = s_tab + tpb * HALF;
  const int tok0 = blockIdx.x * tpb;
  const int ntok = min(tpb, s - tok0);
  const T* xs = (const T*)x + (size_t)tok0 * h * D;
  T* ys = (T*)y + (size_t)tok0 * h * D;
  const int units = ntok * h * GROUPS;

  // unit u = (token, head, group), group fastest; its first pair sits at
  // (u / GROUPS) * D + (u % GROUPS) * 8 from the block's first token
  Piece<BF16> pa[ROPE_UNROLL], pb[ROPE_UNROLL];
  auto load = [&](int u0) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < ROPE_UNROLL; ++r) {
      const int u = u0 + r * ROPE_THREADS;
      if (u < units) {
        const size_t off = (size_t)(u / GROUPS) * D + (u % GROUPS) * 8;
        if constexpr (BF16) {
          pa[r].v = *(const u32x4*)(xs + off);
          pb[r].v = *(const u32x4*)(xs + off + HALF);
        } else {
          pa[r].v[0] = *(const f32x4*)(xs + off);
          pa[r].v[1] = *(const f32x4*)(xs + off + 4);
          pb[r].v[0] = *(const f32x4*)(xs + off + HALF);
          pb[r].v[1] = *(const f32x4*)(xs + off + HALF + 4);
        }
      }
    }
  };

  // the first units' loads are in flight while the angles are computed
  load(threadIdx.x);
  for (int a = threadIdx.x; a < ntok * HALF; a += ROPE_THREADS) {
    const int i = a % HALF;
    const double inv_freq = pow(theta, -2.0 * (double)i / (double)D);
    double sn, cs;
    sincos((double)pos[tok0 + a / HALF] * inv_freq, &sn, &cs);
    s_cos[a] = cs;
    s_sin[a] = inverse ? -sn : sn;
  }
  __syncthreads();

  for (int u0 = threadIdx.x; u0 < units; u0 += ROPE_THREADS * ROPE_UNROLL) {
    if (u0 != (int)threadIdx.x) load(u0);
#pragma unroll
    for (int r = 0; r < ROPE_UNROLL; ++r) {
      const int u = u0 + r * ROPE_THREADS;
      if (u >= units) break;
      const int row = u / GROUPS;  // token-in-block * h + head
      const int i0 = (u % GROUPS) * 8;
      const double* cs = s_cos + (row / h) * HALF + i0;
      const double* sn = s_sin + (row / h) * HALF + i0;
      double a[8], b[8];
      if constexpr (BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          a[2 * w] = bf16_lo(pa[r].v[w]);
          a[2 * w + 1] = bf16_hi(pa[r].v[w]);
          b[2 * w] = bf16_lo(pb[r].v[w]);
          b[2 * w + 1] = bf16_hi(pb[r].v[w]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = pa[r].v[0][e];
          a[4 + e] = pa[r].v[1][e];
          b[e] = pb[r].v[0][e];
          b[4 + e] = pb[r].v[1][e];
        }
      }
      float ra[8], rb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ra[e] = (float)(a[e] * cs[e] - b[e] * sn[e]);
        rb[e] = (float)(b[e] * cs[e] + a[e] * sn[e]);
      }
      const size_t off = (size_t)row * D + i0;
      if constexpr (BF16) {
        u32x4 oa, ob;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          oa[w] = pack_bf16x2(ra[2 * w], ra[2 * w + 1]);
          ob[w] = pack_bf16x2(rb[2 * w], rb[2 * w + 1]);
        }
        *(u32x4*)(ys + off) = oa;
        *(u32x4*)(ys + off + HALF) = ob;
      } else {
        *(f32x4*)(ys + off) = f32x4{ra[0], ra[1], ra[2], ra[3]};
        *(f32x4*)(ys + off + 4) = f32x4{ra[4], ra[5], ra[6], ra[7]};
        *(f32x4*)(ys + off + HALF) = f32x4{rb[0], rb[1], rb[2], rb[3]};
        *(f32x4*)(ys + off + HALF + 4) = f32x4{rb[4], rb[5], rb[6], rb[7]};
      }
    }
  }
}

template <int D>
hipError_t launch_rope_d(const void* x, void* y, bool bf16, const int32_t* pos, int s, int h,
                         double theta, int inverse, hipStream_t stream) {
  constexpr int HALF = D / 2;
  // tokens per block: enough units for every thread to take ROPE_UNROLL of
  // them, at least as many angles as threads, within the LDS table
  const int units_per_token = h * (HALF / 8);
  int tpb = ROPE_THREADS / HALF;
  while (tpb * units_per_token < ROPE_THREADS * ROPE_UNROLL && 2 * tpb * HALF <= ROPE_MAX_ANGLES)
    tpb *= 2;
  const dim3 grid((s + tpb - 1) / tpb);
  const size_t lds = (size_t)tpb * HALF * 2 * sizeof(double);
  if (bf16)
    hipLaunchKernelGGL((rope_kernel<D, true>), grid, dim3(ROPE_THREADS), lds, stream, x, y, pos,
                       s, h, tpb, theta, inverse);
  else
    hipLaunchKernelGGL((rope_kernel<D, false>), grid, dim3(ROPE_THREADS), lds, stream, x, y, pos,
                       s, h, tpb, theta, inverse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const void* x, void* y, bool bf16, const int32_t* pos, int s, int h, int d,
                       double theta, int inverse, hipStream_t stream) {
  return d == 64 ? launch_rope_d<64>(x, y, bf16, pos, s, h, theta, inverse, stream)
                 : launch_rope_d<128>(x, y, bf16, pos, s, h, theta, inverse, stream);
}

}  // namespace mmsp
