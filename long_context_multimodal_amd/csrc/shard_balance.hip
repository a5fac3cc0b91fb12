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
//
// Packed samples (variable-length videos packed with reset attention masks:
// "LongVILA Guide ...", sections "Three-Stage Long-Context Alignment
// Curriculum", stage 3, and "Critical Operational Best Practices"): every
// sample is zigzagged on its own.  A token at offset o of sample s (start
// a_s, block length L_s = len_s / 2P) lies in block b = o / L_s and goes to
// rank b or 2P-1-b; since every earlier sample gave each rank exactly
// 2 L_s' = len_s' / P tokens, its slot inside the rank is a_s / P + (low
// block ? 0 : L_s) + o % L_s.  One thread per token: a fill kernel first sets
// every slot to -1, then tokens of samples with valid boundaries are placed.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace mmsp {

// Scratch of the allocation-free MODALITY balance (mmsp_shard_balance_noalloc):
// the per-block visual counts, then the per-block owners, kNoallocMaxBlocks
// int32 each.  Every device the library runs on holds its own copy until the
// process ends, and every call on that device shares it.  Host code never
// passes this name to a kernel: it is a host-side stand-in, and the device
// address comes from hipGetSymbolAddress (noalloc_balance_scratch below).
static __device__ __align__(256) int32_t scratch[2 * kNoallocMaxBlocks];

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

__global__ void __launch_bounds__(256) fill_kernel(int n, int32_t* __restrict__ a,
                                                   int32_t* __restrict__ b,
                                                   int32_t* __restrict__ c) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  a[i] = -1;
  if (b) b[i] = -1;
  if (c) c[i] = -1;
}

__global__ void __launch_bounds__(256) packed_scatter_kernel(
    int n, int n_ranks, const int32_t* __restrict__ starts, int n_samples,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ token_start) {
  const int pos = blockIdx.x * blockDim.x + threadIdx.x;
  if (pos >= n) return;
  const int P = n_ranks;
  // sample of this position: the last s with starts[s] <= pos
  int lo = 0, hi = n_samples;  // answer in [0, n_samples)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (starts[mid] <= pos) lo = mid; else hi = mid;
  }
  const int a = starts[lo], e = starts[lo + 1];
  // boundaries must be multiples of 2P inside [0, n] with the token inside
  if (a < 0 || e > n || a > pos || pos >= e || a % (2 * P) != 0 || e % (2 * P) != 0) return;
  const int L = (e - a) / (2 * P);
  const int o = pos - a;
  const int b = o / L;
  const int high = b >= P;
  const int r = high ? 2 * P - 1 - b : b;
  const int idx = r * (n / P) + a / P + (high ? L : 0) + (o - b * L);
  perm[idx] = pos;
  if (inv_perm) inv_perm[pos] = idx;
  if (token_start) token_start[idx] = a;
}

// Each rank holds N/P tokens ("LongVILA Guide ...", section "Multi-Modal
// Sequence Parallelism (MM-SP) Mechanics"): the rows its permutation names.
// Token rows moved into shard order (gather: dst[i] = src[rows[i]]) or back
// (scatter: dst[rows[i]] = src[i]).  HBM-bound copy: one wave per row, each
// lane moving 16-byte pieces, four in flight before the first store.  A row
// index outside the indexed tensor gives a zero row (gather) or no write
// (scatter) -- the -1 slots of unplaced packed samples.
template <bool GATHER>
__global__ void __launch_bounds__(256) move_rows_kernel(const u32x4* __restrict__ src,
                                                        const int32_t* __restrict__ rows,
                                                        int64_t n_rows, int64_t indexed_rows,
                                                        int cpr, u32x4* __restrict__ dst) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const int lane = threadIdx.x & 63;
  const int32_t t = rows[r];
  const bool ok = t >= 0 && t < indexed_rows;
  if (!GATHER && !ok) return;
  const u32x4* sp = src + (size_t)(GATHER ? (ok ? t : 0) : r) * cpr;
  u32x4* dp = dst + (size_t)(GATHER ? r : t) * cpr;
  for (int c0 = lane; c0 < cpr; c0 += 64 * 4) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 64 * u;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (ok && c < cpr) v[u] = sp[c];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 64 * u;
      if (c < cpr) dp[c] = v[u];
    }
  }
}

// Precondition check of a position array (and of packed sample starts):
// counts i with pos[i] <= pos[i-1], and with starts: starts[i] > pos[i],
// starts[i] < 0 or starts[i] < starts[i-1].  One counter, zeroed by the first
// kernel (no memset, so the pair may be captured in a graph).
__global__ void zero_counter_kernel(int32_t* __restrict__ count) { *count = 0; }

__global__ void __launch_bounds__(256) check_positions_kernel(const int32_t* __restrict__ pos,
                                                              const int32_t* __restrict__ starts,
                                                              int n, int32_t* __restrict__ count) {
  int bad = 0;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    if (i > 0 && pos[i] <= pos[i - 1]) ++bad;
    if (starts) {
      if (starts[i] > pos[i] || starts[i] < 0) ++bad;
      if (i > 0 && starts[i] < starts[i - 1]) ++bad;
    }
  }
  if (bad) atomicAdd(count, bad);
}

}  // namespace

hipError_t launch_check_positions(const int32_t* pos, const int32_t* starts, int n,
                                  int32_t* count, hipStream_t stream) {
  hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(1), 0, stream, count);
  const int blocks = (int)std::min<int64_t>(1024, ((int64_t)n + 255) / 256);
  hipLaunchKernelGGL(check_positions_kernel, dim3(blocks), dim3(256), 0, stream, pos, starts, n,
                     count);
  return hipGetLastError();
}

hipError_t launch_move_rows(const void* src, const int32_t* rows, int64_t n_rows,
                            int64_t indexed_rows, int64_t row_bytes, void* dst, bool gather,
                            hipStream_t stream) {
  const int cpr = (int)(row_bytes / 16);
  const dim3 grid((unsigned)((n_rows + 3) / 4));
  if (gather)
    hipLaunchKernelGGL(move_rows_kernel<true>, grid, dim3(256), 0, stream, (const u32x4*)src,
                       rows, n_rows, indexed_rows, cpr, (u32x4*)dst);
  else
    hipLaunchKernelGGL(move_rows_kernel<false>, grid, dim3(256), 0, stream, (const u32x4*)src,
                       rows, n_rows, indexed_rows, cpr, (u32x4*)dst);
  return hipGetLastError();
}

hipError_t launch_shard_balance_packed(const int32_t* starts, int n_samples, int n, int n_ranks,
                                       int32_t* perm, int32_t* inv_perm, int32_t* token_start,
                                       hipStream_t stream) {
  const dim3 grid((n + 255) / 256);
  hipLaunchKernelGGL(fill_kernel, grid, dim3(256), 0, stream, n, perm, inv_perm, token_start);
  hipLaunchKernelGGL(packed_scatter_kernel, grid, dim3(256), 0, stream, n, n_ranks, starts,
                     n_samples, perm, inv_perm, token_start);
  return hipGetLastError();
}

hipError_t noalloc_balance_scratch(int32_t** vis, int32_t** owner) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {  // once per device, with that device current
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      addr[dev] = p;
    }
    p = addr[dev];
  }
  *vis = static_cast<int32_t*>(p);
  *owner = static_cast<int32_t*>(p) + kNoallocMaxBlocks;
  return hipSuccess;
}

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
