// Log-sum-exp merge of two chunk results, and the backward preprocess.
//
// Merge: the ring loop of "LongVILA Guide: 2M Context Multi-Modal AI Model",
// section "Implementation: PyTorch Distributed Pipeline and Token Routing",
// accumulates one chunk's attention output per ring step; over disjoint key
// sets the exact accumulation is L = ln(e^La + e^Lb),
// O = e^(La-L) O_a + e^(Lb-L) O_b, with (0, -inf) as identity.
//
// Both kernels are HBM-bound streaming passes: each thread owns 4 consecutive
// fp32 elements of one (token, head) row (16-byte loads/stores); the per-row
// statistics are read once per row by every thread of that row (L1-served).
#include "common.h"
#include "kernels.h"

namespace mmsp {
namespace {

template <int D>
__global__ void __launch_bounds__(256) lse_merge_kernel(float* __restrict__ o_acc,
                                                        float* __restrict__ lse_acc,
                                                        const float* __restrict__ o_part,
                                                        const float* __restrict__ lse_part,
                                                        int sq, int hq,
                                                        uint16_t* __restrict__ o_bf16) {
  constexpr int TPR = D / 4;  // threads per (token, head) row
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long rows = (long long)sq * hq;
  const long long r = idx / TPR;
  if (r >= rows) return;
  const int c4 = (int)(idx % TPR);
  const int i = (int)(r / hq), h = (int)(r % hq);
  float* op = o_acc + r * D + 4 * c4;
  f32x4 oa = *(const f32x4*)op;
  f32x4 out = oa;
  if (o_part != nullptr) {
    const size_t li = (size_t)h * sq + i;
    const float la = lse_acc[li] * kLog2e, lb = lse_part[li] * kLog2e;
    const float mx = fmaxf(la, lb);
    if (mx != -INFINITY) {
      const float ea = fast_exp2(la - mx), eb = fast_exp2(lb - mx);
      const float tot = ea + eb;
      const float wa = ea / tot, wb = eb / tot;
      const f32x4 ob = *(const f32x4*)(o_part + r * D + 4 * c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = fmaf(wa, oa[e], wb * ob[e]);
      *(f32x4*)op = out;
      if (c4 == 0) lse_acc[li] = (mx + __builtin_amdgcn_logf(tot)) * kLn2;
    } else {
      out = f32x4{0.f, 0.f, 0.f, 0.f};
      *(f32x4*)op = out;
      if (c4 == 0) lse_acc[li] = -INFINITY;
    }
  }
  if (o_bf16 != nullptr) {
    u32x2 w = {pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3])};
    *(u32x2*)(o_bf16 + r * D + 4 * c4) = w;
  }
}

// delta[h][i] = sum_c dout[i][h][c] * o[i][h][c]; 16 threads per row, 8 bf16
// of each operand per thread, reduced with cross-lane adds.  Optionally
// zeroes the same 8 elements of the fp32 dQ accumulator.
template <int D>
__global__ void __launch_bounds__(256) bwd_preprocess_kernel(const uint16_t* __restrict__ o,
                                                             const uint16_t* __restrict__ dout,
                                                             int sq, int hq,
                                                             float* __restrict__ delta,
                                                             float* __restrict__ dq_zero) {
  constexpr int TPR = D / 8;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long rows = (long long)sq * hq;
  const long long r = idx / TPR;
  const int c8 = (int)(idx % TPR);
  float acc = 0.f;
  if (r < rows) {
    if (dq_zero != nullptr) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *(f32x4*)(dq_zero + r * D + 8 * c8) = z;
      *(f32x4*)(dq_zero + r * D + 8 * c8 + 4) = z;
    }
    const u32x4 a = *(const u32x4*)(o + r * D + 8 * c8);
    const u32x4 b = *(const u32x4*)(dout + r * D + 8 * c8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16_lo(a[w]), bf16_lo(b[w]), acc);
      acc = fmaf(bf16_hi(a[w]), bf16_hi(b[w]), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (r < rows && c8 == 0) {
    const int i = (int)(r / hq), h = (int)(r % hq);
    delta[(size_t)h * sq + i] = acc;
  }
}

}  // namespace

hipError_t launch_lse_merge(float* o_acc, float* lse_acc, const float* o_part,
                            const float* lse_part, int sq, int hq, int d, uint16_t* o_bf16,
                            hipStream_t stream) {
  const long long threads = (long long)sq * hq * (d / 4);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (d == 64)
    hipLaunchKernelGGL(lse_merge_kernel<64>, dim3(grid), dim3(256), 0, stream, o_acc, lse_acc,
                       o_part, lse_part, sq, hq, o_bf16);
  else
    hipLaunchKernelGGL(lse_merge_kernel<128>, dim3(grid), dim3(256), 0, stream, o_acc, lse_acc,
                       o_part, lse_part, sq, hq, o_bf16);
  return hipGetLastError();
}

hipError_t launch_bwd_preprocess(const uint16_t* o, const uint16_t* dout, int sq, int hq, int d,
                                 float* delta, float* dq_zero, hipStream_t stream) {
  const long long threads = (long long)sq * hq * (d / 8);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (d == 64)
    hipLaunchKernelGGL(bwd_preprocess_kernel<64>, dim3(grid), dim3(256), 0, stream, o, dout, sq,
                       hq, delta, dq_zero);
  else
    hipLaunchKernelGGL(bwd_preprocess_kernel<128>, dim3(grid), dim3(256), 0, stream, o, dout, sq,
                       hq, delta, dq_zero);
  return hipGetLastError();
}

}  // namespace mmsp
