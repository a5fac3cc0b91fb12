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
//  * K/V tiles of 64 keys go straight from HBM to a double-buffered,
//    XOR-swizzled LDS area with 16-byte direct loads (no staging registers);
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: a lane holds 16 scores of ONE
//    query, so the row max/sum are in-lane plus one permlane32 swap;
//  * O^T += V^T P^T: the score registers, converted to bf16, are the B
//    operand in place; V^T comes from the row-major V tile through the
//    transposing LDS read (ds_read_b64_tr_b16);
//  * online softmax in the log2 domain; the running max is only raised when
//    a tile's max exceeds it by more than 8 (2^8 headroom in fp32/bf16), so
//    the O rescale is skipped on most tiles without changing the result;
//    row sums stay in fp32 (exact LSE for the merge and the backward);
//  * causal tile skipping from the sorted positions: a binary search bounds
//    the key range of the workgroup, each wave skips tiles it cannot see and
//    masks only the tiles that straddle its rows' positions;
//  * GQA: query head h reads KV head h / G; the workgroup order keeps the
//    query heads of one KV head on one XCD (shared L2).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mmsp {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int THREADS = 256;
  static constexpr int KS = D / 16;        // K-steps of S^T = K Q^T
  static constexpr int MB = D / 32;        // 32-row blocks of O^T
  static constexpr int NKB = BN / 32;      // 32-key blocks per tile
  static constexpr int TILE = BN * D * 2;  // bytes of one K or V tile
};

template <int D, bool ACC>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(FwdParams p) {
  using C = FwdCfg<D>;
  // one LDS object per pipeline buffer, so the compiler can tell that the
  // direct loads into one buffer never alias reads of the other
  __shared__ __attribute__((aligned(16))) char sK0[C::TILE], sK1[C::TILE];
  __shared__ __attribute__((aligned(16))) char sV0[C::TILE], sV1[C::TILE];
  __shared__ int sKp0[C::BN], sKp1[C::BN];
  auto ktile = [&](auto b) -> lds_char* {
    if constexpr (decltype(b)::value == 0) return (lds_char*)sK0; else return (lds_char*)sK1;
  };
  auto vtile = [&](auto b) -> lds_char* {
    if constexpr (decltype(b)::value == 0) return (lds_char*)sV0; else return (lds_char*)sV1;
  };
  auto kpos_of = [&](auto b) -> int* {
    if constexpr (decltype(b)::value == 0) return sKp0; else return sKp1;
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

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
  wqmin = uniform(wqmin);
  wqmax = uniform(wqmax);
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
  const int nt = uniform((nk + C::BN - 1) / C::BN);

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

  // ---- per-lane LDS offsets (loop invariant) ----
  int koff[C::KS];  // K rows l32 (+32 kb), chunk 2 ks + hh
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) koff[ks] = tile_off<D>(l32, 2 * ks + hh);
  int voff[2][C::MB];  // transposing reads of V: rows 16 ks2 + ..., cols 32 mb + l32
#pragma unroll
  for (int rh = 0; rh < 2; ++rh)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) voff[rh][mb] = tr_offset<D>(lane, 0, rh, mb);

  // ---- tile loads (direct to LDS) ----
  const size_t kv_row_stride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)kvh * D;
  TileLoader<D, C::BN, C::THREADS> ld;
  ld.init(tid, kv_row_stride);
  int kpreg = kPosInf;
  auto issue_tile = [&](int t, auto buf) {
    const int j0 = t * C::BN;
    const size_t o = (size_t)j0 * kv_row_stride;
    if (j0 + C::BN <= p.sk) {
      ld.load(ktile(buf), kbase + o);
      ld.load(vtile(buf), vbase + o);
    } else {
      ld.load_clamped(ktile(buf), kbase + o, kv_row_stride, p.sk - j0);
      ld.load_clamped(vtile(buf), vbase + o, kv_row_stride, p.sk - j0);
    }
    if (tid < C::BN) {
      const int j = j0 + tid;
      kpreg = (j < p.sk) ? (p.causal ? p.k_pos[j] : 0) : kPosInf;
    }
  };

  f32x16 oacc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) oacc[mb] = f32x16{};
  float m_run = -INFINITY;  // running max, log2 domain
  float l_run = 0.f;        // this lane's partial row sum
  const float c = p.scale_log2;

  // one K/V tile; BUF is a compile-time buffer index so every LDS offset is
  // an immediate on top of the per-lane offsets
  auto step = [&](auto buf_tag, int t) {
    constexpr int BUF = decltype(buf_tag)::value;
    using Next = std::integral_constant<int, BUF ^ 1>;
    if (t + 1 < nt) issue_tile(t + 1, Next{});
    const lds_char* kt = ktile(buf_tag);
    const lds_char* vt = vtile(buf_tag);
    const int* kp = kpos_of(buf_tag);
    const int kfirst = uniform(kp[0]);
    const int klast = uniform(kp[C::BN - 1]);
    if (wave_live && kfirst <= wqmax) {
      f32x16 s[C::NKB];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        const int rb = kb * 32 * D * 2;
        s[kb] = mfma32x32x16(lds_read_b128(kt, rb + koff[0]), qf[0], f32x16{});
#pragma unroll
        for (int ks = 1; ks < C::KS; ++ks)
          s[kb] = mfma32x32x16(lds_read_b128(kt, rb + koff[ks]), qf[ks], s[kb]);
      }
      if (klast > wqmin) {  // tile straddles this wave's positions (or the tail)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (kp[key] > qpos) s[kb][i] = -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
      mt = max_halves(mt) * c;
      if (__ballot(mt > m_run + 8.0f)) {
        asm volatile("" ::: "memory");
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) oacc[mb] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
      uint32_t pk[C::NKB][8];
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float e0 = fast_exp2(fmaf(s[kb][i], c, neg_m));
          const float e1 = fast_exp2(fmaf(s[kb][i + 1], c, neg_m));
          pk[kb][i >> 1] = pack_bf16x2(e0, e1);
          if (i & 2) ps1 += e0 + e1; else ps0 += e0 + e1;
        }
      l_run += ps0 + ps1;
#pragma unroll
      for (int ks2 = 0; ks2 < C::BN / 16; ++ks2) {
        const int kb = ks2 >> 1, half = ks2 & 1;
        const u32x4 bw = {pk[kb][4 * half], pk[kb][4 * half + 1], pk[kb][4 * half + 2],
                          pk[kb][4 * half + 3]};
        const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
        const int rb = ks2 * 16 * D * 2;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
          oacc[mb] = mfma32x32x16(lds_read_tr(vt, rb + voff[0][mb], rb + voff[1][mb]), b,
                                  oacc[mb]);
      }
    }
    if (t + 1 < nt) {
      if (tid < C::BN) kpos_of(Next{})[tid] = kpreg;
      wait_vmem();
    }
    __syncthreads();
  };

  if (nt > 0) {
    issue_tile(0, B0{});
    if (tid < C::BN) sKp0[tid] = kpreg;
    wait_vmem();
  }
  __syncthreads();
  for (int t = 0; t < nt; t += 2) {
    step(B0{}, t);
    if (t + 1 < nt) step(B1{}, t + 1);
  }

  // ---- epilogue: normalise, then write or merge ----
  const float l_tot = sum_halves(l_run);
  if (!row_ok) return;
  const bool has = l_tot > 0.f;
  const float inv = has ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
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
    const float rt = __builtin_amdgcn_rcpf(tot);
    const float wa = ea * rt, wb = eb * rt * inv;
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

template __global__ void attn_fwd_kernel<64, false>(FwdParams);
template __global__ void attn_fwd_kernel<64, true>(FwdParams);
template __global__ void attn_fwd_kernel<128, false>(FwdParams);
template __global__ void attn_fwd_kernel<128, true>(FwdParams);

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
