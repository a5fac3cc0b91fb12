// Shard permutation giving every rank equal causal work (integer, bit-exact).
//
// Problem: modality-switching boundaries leave one rank with text and another
// with dense visual tokens ("LongVILA Guide: 2M Context Multi-Modal AI
// Model", section "Problem", item 2); work is dispatched by modality token
// density ("Ultra-Large Multimodal LLM Inference ...", section 4, "Load
// Balancing for Tensor Parallelism").  Under a causal mask position p costs
// p + 1 key visits, so the stream is cut into blocks of g tokens and each
// round of 2P blocks is paired outside-in (blocks 2jP+a and 2jP+2P-1-a); all
// pairs of a round cost the same, so every rank gets the same work whatever
// the assignment.  ZIGZAG is the one-round case with pair a -> rank a;
// MODALITY hands the pairs, in order of decreasing visual count, to the ranks
// in order of increasing running visual total (ties to the lower index).
//
// Kernels: (1) visual count per block (one wave per block); (2) the
// sequential-over-rounds assignment in one workgroup, pair and rank orders
// found by counting comparisons in parallel; (3) a scatter of every token to
// its rank-major slot.  A rank owns exactly one low and one high block per
// round, so a block's slot inside its rank is 2*round + (high half ? 1 : 0).
#include "common.h"
#include "kernels.h"

namespace mmsp {
namespace {

__global__ void __launch_bounds__(64) block_visual_kernel(const uint8_t* __restrict__ labels,
                                                          int g, int32_t* __restrict__ vis) {
  const int b = blockIdx.x;
  const uint8_t* lb = labels + (size_t)b * g;
  int cnt = 0;
  for (int t = threadIdx.x; t < g; t += 64) cnt += (lb[t] != 0);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
  if (threadIdx.x == 0) vis[b] = cnt;
}

__global__ void __launch_bounds__(1024) modality_assign_kernel(const int32_t* __restrict__ vis,
                                                               int32_t* __restrict__ owner,
                                                               int n_ranks, int rounds) {
  __shared__ int pv[1024], cum[1024], pair_at[1024], rank_at[1024];
  const int t = threadIdx.x;
  const int P = n_ranks;
  if (t < P) cum[t] = 0;
  __syncthreads();
  for (int j = 0; j < rounds; ++j) {
    const int base = 2 * j * P;
    if (t < P) pv[t] = vis[base + t] + vis[base + 2 * P - 1 - t];
    __syncthreads();
    if (t < P) {
      const int my_pv = pv[t], my_cum = cum[t];
      int kp = 0, kr = 0;
      for (int a = 0; a < P; ++a) {
        const int o = pv[a];
        kp += (o > my_pv) || (o == my_pv && a < t);
        const int c = cum[a];
        kr += (c < my_cum) || (c == my_cum && a < t);
      }
      pair_at[kp] = t;
      rank_at[kr] = t;
    }
    __syncthreads();
    if (t < P) {
      const int a = pair_at[t], r = rank_at[t];
      owner[base + a] = r;
      owner[base + 2 * P - 1 - a] = r;
      cum[r] += pv[a];
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) scatter_kernel(int n, int n_ranks, int g, int zigzag,
                                                      const int32_t* __restrict__ owner,
                                                      int32_t* __restrict__ perm,
                                                      int32_t* __restrict__ inv_perm) {
  const int pos = blockIdx.x * blockDim.x + threadIdx.x;
  if (pos >= n) return;
  const int P = n_ranks;
  const int b = pos / g;
  const int j = b / (2 * P);
  const int ab = b - j * 2 * P;
  const int hi = ab >= P;
  const int r = zigzag ? (hi ? 2 * P - 1 - ab : ab) : owner[b];
  const int shard = n / P;
  const int idx = r * shard + (2 * j + hi) * g + (pos - b * g);
  perm[idx] = pos;
  if (inv_perm) inv_perm[pos] = idx;
}

}  // namespace

hipError_t launch_shard_balance(const uint8_t* labels, int n, int n_ranks, int mode, int g,
                                int32_t* perm, int32_t* inv_perm, int32_t* ws_vis,
                                int32_t* ws_owner, hipStream_t stream) {
  const bool zig = mode == 0;
  if (zig) g = n / (2 * n_ranks);
  if (!zig) {
    const int n_blocks = n / g;
    const int rounds = n_blocks / (2 * n_ranks);
    hipLaunchKernelGGL(block_visual_kernel, dim3(n_blocks), dim3(64), 0, stream, labels, g,
                       ws_vis);
    const int threads = ((n_ranks + 63) / 64) * 64;
    hipLaunchKernelGGL(modality_assign_kernel, dim3(1), dim3(threads), 0, stream, ws_vis,
                       ws_owner, n_ranks, rounds);
  }
  hipLaunchKernelGGL(scatter_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, n, n_ranks, g,
                     zig ? 1 : 0, ws_owner, perm, inv_perm);
  return hipGetLastError();
}

}  // namespace mmsp
