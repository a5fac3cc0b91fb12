// Work-ordered tile lists for the packed attention kernels.
//
// With packed samples ("LongVILA Guide: 2M Context Multi-Modal AI Model",
// section "Critical Operational Best Practices": several videos share one
// buffer, with reset attention masks) the work of a workgroup varies with the
// samples its tile holds: a query tile whose rows start a sample sees few
// keys, one at the end of a long sample sees many, and a key tile past every
// sample start of the shard sees none.  The kernels' built-in order assumes
// the plain causal shape (work growing with the tile index), which for packed
// shards leaves the heaviest tiles to the last round of workgroups.  These
// kernels count each tile's work from the positions, with the same ranges the
// attention kernels compute, and list the tiles heaviest first (longest
// processing time first list scheduling); the attention kernels then take
// their tiles from the lists.  Any order gives the same results bit for bit:
// each workgroup's arithmetic does not depend on when it runs.
#include "common.h"
#include "kernels.h"

namespace mmsp {
namespace {

struct PlanArgs {
  const int32_t* q_pos;
  const int32_t* q_start;
  const int32_t* k_pos;
  int sq, sk;
  int fwd_bm, fwd_bn;    // forward: query rows per workgroup, keys per tile
  int dq_bm, dq_bn;      // dQ kernel: query rows per workgroup, keys per tile
  int dkdv_bk, dkdv_bq;  // dK/dV kernel: keys per workgroup, query rows per tile
  int n_fwd, n_dq, n_dkdv;
  int fwd_off, dq_off, dkdv_off, work_off;
  int32_t* plan;
  int plan_words;  // stride of consecutive plans (several chunks in one launch)
};

// Entries of the non-decreasing array a[0, n) below xa, and of b[0, n) at or
// below xb: two branch-free binary searches stepped together, so each level
// costs one memory round trip for both.
__device__ __forceinline__ void count_two(const int32_t* a, int xa, const int32_t* b, int xb,
                                          int n, int& ca, int& cb) {
  int step = 1;
  while (step <= n) step <<= 1;
  int pa = 0, pb = 0;
  for (step >>= 1; step > 0; step >>= 1) {
    if (pa + step <= n && a[pa + step - 1] < xa) pa += step;
    if (pb + step <= n && b[pb + step - 1] <= xb) pb += step;
  }
  ca = pa;
  cb = pb;
}

// Work of tile i (all three sections numbered together), in tiles of the
// kernel's inner loop: key tiles for the query-stationary forward and dQ
// kernels (from the first key at or after the tile's smallest sample start to
// the last key at or before its largest position), query tiles for the
// key-stationary dK/dV kernel (from the first query at or after the tile's
// smallest key position to the last query whose sample starts at or before
// its largest one).  The position arrays may sit in global memory or in LDS.
__device__ __forceinline__ int tile_work(const PlanArgs& a, const int32_t* q_pos,
                                         const int32_t* q_start, const int32_t* k_pos, int i) {
  if (i < a.n_fwd + a.n_dq) {
    const bool fwd = i < a.n_fwd;
    const int t = fwd ? i : i - a.n_fwd;
    const int bm = fwd ? a.fwd_bm : a.dq_bm, bn = fwd ? a.fwd_bn : a.dq_bn;
    const int q0 = t * bm;
    const int qmax = q_pos[min(q0 + bm - 1, a.sq - 1)];
    int kbeg, nk;
    count_two(k_pos, q_start[q0], k_pos, qmax, a.sk, kbeg, nk);
    return max(0, (nk + bn - 1) / bn - kbeg / bn);
  }
  const int t = i - a.n_fwd - a.n_dq;
  const int j0 = t * a.dkdv_bk;
  const int kmin = k_pos[j0], kmax = k_pos[min(j0 + a.dkdv_bk - 1, a.sk - 1)];
  int qbeg, qend;
  count_two(q_pos, kmin, q_start, kmax, a.sq, qbeg, qend);
  return max(0, (qend + a.dkdv_bq - 1) / a.dkdv_bq - qbeg / a.dkdv_bq);
}

__device__ __forceinline__ void write_header(const PlanArgs& a) {
  a.plan[0] = kPlanMagic;
  a.plan[1] = a.sq;
  a.plan[2] = a.sk;
  a.plan[3] = a.n_fwd;
  a.plan[4] = a.n_dq;
  a.plan[5] = a.n_dkdv;
  a.plan[6] = 0;
  a.plan[7] = 0;
}

// Shards of at most kSmallPlan positions (the usual case): one workgroup per
// chunk stages the three position arrays in LDS, counts every tile's work
// there and ranks the tiles; the chunks of one launch have consecutive key
// positions (sk apart) and consecutive plans (plan_words apart).
constexpr int kSmallPlan = 8192;
constexpr int kSmallThreads = 1024;

__global__ void __launch_bounds__(kSmallThreads) plan_small_kernel(PlanArgs args) {
  __shared__ int32_t s_q[kSmallPlan], s_s[kSmallPlan], s_k[kSmallPlan];
  __shared__ int32_t s_w[kSmallThreads];
  PlanArgs a = args;
  a.k_pos += (size_t)blockIdx.x * a.sk;
  a.plan += (size_t)blockIdx.x * a.plan_words;
  const int tid = threadIdx.x;
  // every load issued before the first store: one memory round trip
  constexpr int PER = kSmallPlan / kSmallThreads;
  int32_t rk[PER], rq[PER], rs[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * kSmallThreads;
    rk[u] = i < a.sk ? a.k_pos[i] : 0;
    rq[u] = i < a.sq ? a.q_pos[i] : 0;
    rs[u] = i < a.sq ? a.q_start[i] : 0;
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * kSmallThreads;
    s_k[i] = rk[u];
    s_q[i] = rq[u];
    s_s[i] = rs[u];
  }
  __syncthreads();
  const int total = a.n_fwd + a.n_dq + a.n_dkdv;  // <= kSmallThreads for these sizes
  const int w = tid < total ? tile_work(a, s_q, s_s, s_k, tid) : -1;
  s_w[tid] = w;
  __syncthreads();
  if (tid < total) {
    a.plan[a.work_off + tid] = w;
    // rank within the section: descending work, ties by ascending index
    const int sec = tid < a.n_fwd ? 0 : tid < a.n_fwd + a.n_dq ? 1 : 2;
    const int b = sec == 0 ? 0 : sec == 1 ? a.n_fwd : a.n_fwd + a.n_dq;
    const int n = sec == 0 ? a.n_fwd : sec == 1 ? a.n_dq : a.n_dkdv;
    const int list = sec == 0 ? a.fwd_off : sec == 1 ? a.dq_off : a.dkdv_off;
    int rank = 0;
    for (int j = b; j < b + n; ++j) {
      const int wj = s_w[j];
      rank += (wj > w) || (wj == w && j < tid);
    }
    a.plan[list + rank] = tid - b;
  }
  if (tid == 0) write_header(a);
}

// Larger shards: one thread per tile counts its work from global memory ...
__global__ void __launch_bounds__(256) plan_work_kernel(PlanArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.n_fwd + a.n_dq + a.n_dkdv) return;
  a.plan[a.work_off + i] = tile_work(a, a.q_pos, a.q_start, a.k_pos, i);
}

// Sections longer than this keep index order: ranking costs n^2 compares.
constexpr int kMaxRanked = 1 << 15;

// ... then one thread per tile of section blockIdx.y finds its rank among the
// section's tiles by descending work, ties by ascending index: its slot in
// the list.
__global__ void __launch_bounds__(256) plan_order_kernel(PlanArgs a) {
  __shared__ int sw[256];
  const int sec = blockIdx.y;
  const int n = sec == 0 ? a.n_fwd : sec == 1 ? a.n_dq : a.n_dkdv;
  const int list = sec == 0 ? a.fwd_off : sec == 1 ? a.dq_off : a.dkdv_off;
  const int work = a.work_off + (sec == 0 ? 0 : sec == 1 ? a.n_fwd : a.n_fwd + a.n_dq);
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.x * blockDim.x >= n) return;  // whole block past the section
  if (n > kMaxRanked) {
    if (i < n) a.plan[list + i] = i;
  } else {
    const int wi = i < n ? a.plan[work + i] : 0;
    int rank = 0;
    for (int base = 0; base < n; base += 256) {
      const int j = base + (int)threadIdx.x;
      sw[threadIdx.x] = j < n ? a.plan[work + j] : -1;  // -1: below every work
      __syncthreads();
      const int m = min(256, n - base);
      for (int k = 0; k < m; ++k) {
        const int wj = sw[k];
        rank += (wj > wi) || (wj == wi && base + k < i);
      }
      __syncthreads();
    }
    if (i < n) a.plan[list + rank] = i;
  }
  if (sec == 0 && i == 0) write_header(a);
}

}  // namespace

PlanShape plan_shape(int sq, int sk) {
  const int fb = fwd_rows_per_block(), qb = bwd_rows_per_block(), kb = bwd_keys_per_block();
  return PlanShape{(sq + fb - 1) / fb, (sq + qb - 1) / qb, (sk + kb - 1) / kb};
}

hipError_t launch_tile_plan(const int32_t* q_pos, const int32_t* q_start, const int32_t* k_pos,
                            int n_chunks, int sq, int sk, int32_t* plan, hipStream_t stream) {
  const PlanShape s = plan_shape(sq, sk);
  PlanArgs a;
  a.q_pos = q_pos;
  a.q_start = q_start;
  a.k_pos = k_pos;
  a.sq = sq;
  a.sk = sk;
  a.fwd_bm = fwd_rows_per_block();
  a.fwd_bn = fwd_keys_per_tile();
  a.dq_bm = bwd_rows_per_block();
  a.dq_bn = dq_keys_per_tile();
  a.dkdv_bk = bwd_keys_per_block();
  a.dkdv_bq = dkdv_rows_per_tile();
  a.n_fwd = s.n_fwd;
  a.n_dq = s.n_dq;
  a.n_dkdv = s.n_dkdv;
  a.fwd_off = s.fwd_off();
  a.dq_off = s.dq_off();
  a.dkdv_off = s.dkdv_off();
  a.work_off = s.work_off();
  a.plan = plan;
  a.plan_words = (int)(s.bytes() / 4);
  const int total = s.n_fwd + s.n_dq + s.n_dkdv;
  if (sq <= kSmallPlan && sk <= kSmallPlan && total <= kSmallThreads) {
    hipLaunchKernelGGL(plan_small_kernel, dim3(n_chunks), dim3(kSmallThreads), 0, stream, a);
    return hipGetLastError();
  }
  const int nmax = max(s.n_fwd, max(s.n_dq, s.n_dkdv));
  for (int c = 0; c < n_chunks; ++c) {
    PlanArgs b = a;
    b.k_pos = k_pos + (size_t)c * sk;
    b.plan = plan + (size_t)c * a.plan_words;
    hipLaunchKernelGGL(plan_work_kernel, dim3((total + 255) / 256), dim3(256), 0, stream, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(plan_order_kernel, dim3((nmax + 255) / 256, 3), dim3(256), 0, stream, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mmsp
