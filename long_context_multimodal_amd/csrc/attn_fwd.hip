// Forward of causal attention of a query shard against one KV chunk (gfx950).
//
// Source of the computation: "LongVILA Guide: 2M Context Multi-Modal AI
// Model", section "Multi-Modal Sequence Parallelism (MM-SP) Mechanics" (one
// attention kernel per ring step on the KV chunk that just arrived) and
// section "Implementation: PyTorch Distributed Pipeline and Token Routing"
// (scores = q.k / sqrt(head_dim), softmax, weighted sum of V, accumulated
// over ring steps).  The accumulation is done exactly with the chunk's
// log-sum-exp (MMSP_ACCUMULATE merges in the epilogue).
//
// Design (one workgroup = 128 query rows of one query head, 4 waves):
//  * each wave owns 32 query rows; Q stays in registers for the whole loop;
//  * K/V tiles of 64 keys are loaded with 16-byte coalesced global loads,
//    prefetched into registers one tile ahead and stored to a double-buffered
//    LDS area (K row-major, V transposed with the key order of kPerm16);
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: a lane holds 16 scores of ONE
//    query, so the row max/sum are in-lane plus one permlane32 swap;
//  * O^T += V^T P^T reuses the score registers (converted to bf16) as the B
//    operand without any data movement;
//  * online softmax in the log2 domain; the running max is only raised when
//    a tile's max exceeds it by more than 8 (2^8 headroom in fp32/bf16), so
//    the O rescale is skipped on most tiles without changing the result;
//  * causal tile skipping from the sorted positions: a binary search bounds
//    the key range of the workgroup, each wave skips tiles it cannot see and
//    masks only the tiles that straddle its rows' positions;
//  * GQA: query head h reads KV head h / G; the workgroup order keeps the
//    query heads of one KV head on one XCD (shared L2).
#include "common.h"
#include "kernels.h"

namespace mmsp {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int THREADS = 256;
  static constexpr int KSTR = D + 8;       // bf16 per K row in LDS (16-byte pad)
  static constexpr int VSTR = BN + 8;      // bf16 per V^T row in LDS
  static constexpr int KS = D / 16;        // K-steps of S^T = K Q^T
  static constexpr int MB = D / 32;        // 32-row blocks of O^T
  static constexpr int CPR = D / 8;        // 16-byte chunks per K/V row
  static constexpr int K_LOADS = BN * CPR / THREADS;
  static constexpr int V_ITEMS = (BN / 4) * CPR;  // (4 keys x 8 dims) items
  static constexpr int NKB = BN / 32;      // 32-key blocks per tile
};

constexpr int kPosInf = 0x7fffffff;

template <int D, bool ACC>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(FwdParams p) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][C::BN * C::KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * C::VSTR];
  __shared__ int sKp[2][C::BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int h = logical / p.n_qtiles;
  const int qt = p.n_qtiles - 1 - (logical % p.n_qtiles);  // late (heavier) tiles first
  const int kvh = h / p.group;
  const int q0 = qt * C::BM;
  const int row = q0 + wave * 32 + l32;
  const bool row_ok = row < p.sq;

  // ---- positions of this lane, this wave and this workgroup ----
  int qpos = INT_MIN;
  if (row_ok) qpos = p.causal ? p.q_pos[row] : (kPosInf - 1);
  const int wr0 = q0 + wave * 32;
  const bool wave_live = wr0 < p.sq;
  int wqmin = 0, wqmax = INT_MIN;
  if (wave_live) {
    const int wlast = min(wr0 + 31, p.sq - 1);
    wqmin = p.causal ? p.q_pos[wr0] : (kPosInf - 1);
    wqmax = p.causal ? p.q_pos[wlast] : (kPosInf - 1);
  }
  int nk = p.sk;
  if (p.causal) {
    const int qmax = p.q_pos[min(q0 + C::BM - 1, p.sq - 1)];
    int lo = 0, hi = p.sk;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (p.k_pos[mid] <= qmax) lo = mid + 1; else hi = mid;
    }
    nk = lo;
  }
  const int nt = (nk + C::BN - 1) / C::BN;

  // ---- Q fragment: B operand of S^T = K Q^T (col = query, k = head dim) ----
  bf16x8 qf[C::KS];
  {
    const uint16_t* qp = p.q + ((size_t)row * p.hq + h) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row_ok) w = *(const u32x4*)(qp + 16 * ks);
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- tile staging: global -> registers (prefetch) -> LDS ----
  u32x4 kreg[C::K_LOADS];
  u32x4 vreg[4];
  int kpreg = kPosInf;
  const size_t kv_row_stride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)kvh * D;

  auto load_tile = [&](int t) {
    const int j0 = t * C::BN;
#pragma unroll
    for (int c = 0; c < C::K_LOADS; ++c) {
      const int idx = tid + c * C::THREADS;
      const int r = idx / C::CPR, cc = idx % C::CPR;
      const int j = j0 + r;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (j < p.sk) w = *(const u32x4*)(kbase + (size_t)j * kv_row_stride + cc * 8);
      kreg[c] = w;
    }
    if (tid < C::V_ITEMS) {
      const int kg = tid / C::CPR, dc = tid % C::CPR;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * kg + r;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (j < p.sk) w = *(const u32x4*)(vbase + (size_t)j * kv_row_stride + dc * 8);
        vreg[r] = w;
      }
    }
    if (tid < C::BN) {
      const int j = j0 + tid;
      kpreg = (j < p.sk) ? (p.causal ? p.k_pos[j] : 0) : kPosInf;
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < C::K_LOADS; ++c) {
      const int idx = tid + c * C::THREADS;
      const int r = idx / C::CPR, cc = idx % C::CPR;
      *(u32x4*)&sK[buf][r * C::KSTR + cc * 8] = kreg[c];
    }
    if (tid < C::V_ITEMS) {
      const int kg = tid / C::CPR, dc = tid % C::CPR;
      const int key = 4 * kg;
      const int col = (key & ~15) + kPerm16(key & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t a0 = vreg[0][w], a1 = vreg[1][w], a2 = vreg[2][w], a3 = vreg[3][w];
        u32x2 out;
        if ((e & 1) == 0) {
          out[0] = (a0 & 0xffffu) | (a1 << 16);
          out[1] = (a2 & 0xffffu) | (a3 << 16);
        } else {
          out[0] = (a0 >> 16) | (a1 & 0xffff0000u);
          out[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        }
        *(u32x2*)&sV[buf][(8 * dc + e) * C::VSTR + col] = out;
      }
    }
    if (tid < C::BN) sKp[buf][tid] = kpreg;
  };

  f32x16 oacc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) oacc[mb] = f32x16{};
  float m_run = -INFINITY;  // running max, log2 domain
  float l_run = 0.f;        // this lane's partial row sum
  const float c = p.scale_log2;

  if (nt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nt) load_tile(t + 1);
    const int kfirst = sKp[buf][0];
    const int klast = sKp[buf][C::BN - 1];
    if (wave_live && kfirst <= wqmax) {
      const bool full = klast <= wqmin;
      f32x16 s[C::NKB];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        s[kb] = f32x16{};
        const uint16_t* kr = &sK[buf][(kb * 32 + l32) * C::KSTR + 8 * hh];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(kr + 16 * ks));
          s[kb] = mfma32x32x16(a, qf[ks], s[kb]);
        }
      }
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (sKp[buf][key] > qpos) s[kb][i] = -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
      mt = max_halves(mt) * c;
      if (__ballot(mt > m_run + 8.0f)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) oacc[mb] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
      uint32_t pk[C::NKB][8];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float e0 = fast_exp2(fmaf(s[kb][i], c, neg_m));
          const float e1 = fast_exp2(fmaf(s[kb][i + 1], c, neg_m));
          psum += e0 + e1;
          pk[kb][i >> 1] = pack_bf16x2(e0, e1);
        }
      l_run += psum;
#pragma unroll
      for (int ks2 = 0; ks2 < C::BN / 16; ++ks2) {
        const int kb = ks2 >> 1, half = ks2 & 1;
        const u32x4 bw = {pk[kb][4 * half], pk[kb][4 * half + 1], pk[kb][4 * half + 2],
                          pk[kb][4 * half + 3]};
        const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
        const uint16_t* vr = &sV[buf][l32 * C::VSTR + 16 * ks2 + 8 * hh];
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(vr + mb * 32 * C::VSTR));
          oacc[mb] = mfma32x32x16(a, b, oacc[mb]);
        }
      }
    }
    if (t + 1 < nt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, then write or merge ----
  const float l_tot = sum_halves(l_run);
  if (!row_ok) return;
  const bool has = l_tot > 0.f;
  const float inv = has ? 1.f / l_tot : 0.f;
  const float lse2 = has ? m_run + __builtin_amdgcn_logf(l_tot) : -INFINITY;  // log2 domain
  float* orow = p.o + ((size_t)row * p.hq + h) * D;
  float* lrow = p.lse + (size_t)h * p.sq + row;
  if (!ACC) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * hh;
        f32x4 val = {oacc[mb][4 * g] * inv, oacc[mb][4 * g + 1] * inv,
                     oacc[mb][4 * g + 2] * inv, oacc[mb][4 * g + 3] * inv};
        *(f32x4*)(orow + d0) = val;
      }
    if (hh == 0) *lrow = has ? lse2 * kLn2 : -INFINITY;
  } else {
    if (!has) return;  // merging with an empty result is the identity
    const float la2 = *lrow * kLog2e;  // -inf stays -inf
    const float mx = fmaxf(la2, lse2);
    const float ea = fast_exp2(la2 - mx), eb = fast_exp2(lse2 - mx);
    const float tot = ea + eb;
    const float wa = ea / tot, wb = eb / tot * inv;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * hh;
        const f32x4 old = *(const f32x4*)(orow + d0);
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = fmaf(wa, old[e], wb * oacc[mb][4 * g + e]);
        *(f32x4*)(orow + d0) = val;
      }
    if (hh == 0) *lrow = (mx + __builtin_amdgcn_logf(tot)) * kLn2;
  }
}

template <int D>
hipError_t launch_fwd_d(const FwdParams& p, hipStream_t stream) {
  const int grid = p.n_qtiles * p.hq;
  if (p.accumulate)
    hipLaunchKernelGGL((attn_fwd_kernel<D, true>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, false>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int fwd_rows_per_block() { return FwdCfg<128>::BM; }

hipError_t launch_attn_fwd(const FwdParams& p, int d, hipStream_t stream) {
  return d == 64 ? launch_fwd_d<64>(p, stream) : launch_fwd_d<128>(p, stream);
}

}  // namespace mmsp
