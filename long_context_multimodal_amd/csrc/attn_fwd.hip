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
// Design (one workgroup = 256 query rows of one query head, 8 waves, two
// waves per SIMD):
//  * each wave owns 32 query rows; Q stays in registers; the 8 waves share
//    every K/V tile, so each tile crosses HBM/L2 -> LDS once per 256 rows;
//  * K/V tiles of 64 keys go straight from HBM to a 4-stage, XOR-swizzled
//    LDS ring with 16-byte direct loads (no staging registers), three tiles
//    in flight ahead of the one being used; each stage
//    is its own LDS object so loads into one never stall reads of another;
//    the key positions of a tile are loaded directly into a per-wave slot;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: a lane holds 16 scores of ONE
//    query, so the row max/sum are in-lane plus one permlane32 swap;
//  * O^T += V^T P^T: the score registers, converted to bf16, are the B
//    operand in place; V^T comes from the row-major V tile through the
//    transposing LDS read (ds_read_b64_tr_b16);
//  * online softmax in the log2 domain; the running max is only raised when
//    a tile's max exceeds it by more than 8 (2^8 headroom in fp32/bf16), so
//    the O rescale is skipped on most tiles without changing the result;
//    on unmasked tiles of rows that already have a running max the tile max
//    is not even computed: weights are taken against the running max, and a
//    lane row sum above 2^16 (a row max more than 16 above it) sends the
//    tile back through the max-and-rescale path, its scores recomputed from
//    the K tile still in LDS; row sums stay in fp32 (exact LSE for the
//    merge and the backward);
//  * causal tile skipping from the sorted positions: a binary search bounds
//    the key range of the workgroup, each wave skips tiles it cannot see and
//    masks only the tiles that straddle its rows' positions (or the tail),
//    with one unsigned compare per score (sample start <= key position <=
//    query position);
//  * packed samples (reset masks between samples packed in one buffer) take
//    a per-query sample start that also bounds the key range from below;
//    they run in their own template instance, so the plain path has none of
//    that code;
//  * GQA: query head h reads KV head h / G; the workgroup order keeps the
//    query heads of one KV head on one XCD (shared L2) and dispatches the
//    heavier (causally longer) query tiles first; when one head's tiles span
//    several XCDs, heavy and light tiles alternate in blocks of 8 so every
//    XCD and shader engine gets an even share.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mmsp {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 512;
  static constexpr int QB = 1;                // 32-row query blocks per wave
  static constexpr int BM = WAVES * 32 * QB;  // query rows per workgroup
  static constexpr int BN = 64;               // keys per tile
  static constexpr int NS = 4;                // pipeline stages (K/V tiles in flight + 1)
  static constexpr int KS = D / 16;           // K-steps of S^T = K Q^T
  static constexpr int MB = D / 32;           // 32-row blocks of O^T
  static constexpr int NKB = BN / 32;         // 32-key blocks per tile
  static constexpr int TILE = BN * D * 2;     // bytes of one K or V tile
  using Loader = TileLoader<D, BN, THREADS>;
  static constexpr int VMEM = 2 * Loader::ROUNDS + 1;  // vector-memory ops per tile per thread
};

template <int D, bool ACC, bool PACKED>
__global__ void __launch_bounds__(512, 1) attn_fwd_kernel(FwdParams p) {
  using C = FwdCfg<D>;
  // one LDS object per pipeline stage
  static_assert(C::NS == 4, "stage objects below are written out for four stages");
  __shared__ __attribute__((aligned(16))) char sK0[C::TILE], sK1[C::TILE], sK2[C::TILE],
      sK3[C::TILE];
  __shared__ __attribute__((aligned(16))) char sV0[C::TILE], sV1[C::TILE], sV2[C::TILE],
      sV3[C::TILE];
  __shared__ __attribute__((aligned(16))) int sP0[C::WAVES * C::BN], sP1[C::WAVES * C::BN],
      sP2[C::WAVES * C::BN], sP3[C::WAVES * C::BN];
  auto ktile = [&](auto b) -> lds_char* {
    constexpr int S = decltype(b)::value;
    if constexpr (S == 0) return (lds_char*)sK0;
    else if constexpr (S == 1) return (lds_char*)sK1;
    else if constexpr (S == 2) return (lds_char*)sK2;
    else return (lds_char*)sK3;
  };
  auto vtile = [&](auto b) -> lds_char* {
    constexpr int S = decltype(b)::value;
    if constexpr (S == 0) return (lds_char*)sV0;
    else if constexpr (S == 1) return (lds_char*)sV1;
    else if constexpr (S == 2) return (lds_char*)sV2;
    else return (lds_char*)sV3;
  };
  auto ptile = [&](auto b) -> int* {
    constexpr int S = decltype(b)::value;
    if constexpr (S == 0) return sP0;
    else if constexpr (S == 1) return sP1;
    else if constexpr (S == 2) return sP2;
    else return sP3;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int h = logical / p.n_qtiles;
  const int qt = heavy_first_tile(logical % p.n_qtiles, p.n_qtiles, gridDim.x);
  const int kvh = h / p.group;
  const int q0 = qt * C::BM;
  const int wr0 = q0 + wave * 32 * C::QB;  // first row of this wave

  // ---- positions: per lane and block, per block range, workgroup range ----
  int row[C::QB], qpos[C::QB], bmin[C::QB];
  bool row_ok[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    row[qb] = wr0 + 32 * qb + l32;
    row_ok[qb] = row[qb] < p.sq;
    qpos[qb] = INT_MIN;
    if (row_ok[qb]) qpos[qb] = p.causal ? p.q_pos[row[qb]] : (kPosInf - 1);
    const int r0 = wr0 + 32 * qb;
    bmin[qb] = uniform(r0 < p.sq ? (p.causal ? p.q_pos[r0] : (kPosInf - 1)) : kPosInf);
  }
  const bool wave_live = wr0 < p.sq;
  const int wqmax =
      uniform(wave_live ? (p.causal ? p.q_pos[min(wr0 + 32 * C::QB - 1, p.sq - 1)] : kPosInf - 1)
                        : INT_MIN);
  // packed samples: keys below a row's sample start are hidden too
  // (q_start is non-decreasing along the rows, like the positions)
  constexpr bool packed = PACKED;  // q_start given
  int qs[C::QB], bqs_max[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    qs[qb] = (packed && row_ok[qb]) ? p.q_start[row[qb]] : INT_MIN;
    const int r0 = wr0 + 32 * qb;
    bqs_max[qb] = uniform((packed && r0 < p.sq) ? p.q_start[min(r0 + 31, p.sq - 1)] : INT_MIN);
  }
  const int wqs_min = uniform((packed && wave_live) ? p.q_start[wr0] : INT_MIN);
  // key range of the workgroup: [kbeg, nk)
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
  int kbeg = 0;
  if (packed) {
    const int qsmin = p.q_start[q0];
    int lo = 0, hi = p.sk;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (p.k_pos[mid] < qsmin) lo = mid + 1; else hi = mid;
    }
    kbeg = lo;
  }
  const int tb = uniform(kbeg / C::BN);  // first tile
  const int nt = uniform(max(0, (nk + C::BN - 1) / C::BN - tb));

  // ---- Q fragments: B operands of S^T = K Q^T (col = query, k = head dim) ----
  bf16x8 qf[C::QB][C::KS];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const uint16_t* qp = p.q + ((size_t)row[qb] * p.hq + h) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row_ok[qb]) w = *(const u32x4*)(qp + 16 * ks);
      qf[qb][ks] = __builtin_bit_cast(bf16x8, w);
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
  // without a causal mask positions are unused; any readable int array will do
  const int32_t* pos_src = p.causal ? p.k_pos : (const int32_t*)p.k;
  typename C::Loader ld;
  ld.init(tid, kv_row_stride);
  auto issue_tile = [&](int t, auto stage) {
    const int j0 = (tb + t) * C::BN;
    const size_t o = (size_t)j0 * kv_row_stride;
    if (j0 + C::BN <= p.sk) {
      ld.load(ktile(stage), kbase + o);
      ld.load(vtile(stage), vbase + o);
    } else {
      ld.load_clamped(ktile(stage), kbase + o, kv_row_stride, p.sk - j0);
      ld.load_clamped(vtile(stage), vbase + o, kv_row_stride, p.sk - j0);
    }
    pos_load_direct((lds_char*)(ptile(stage) + wave * C::BN), pos_src, j0,
                    min(C::BN, p.sk - j0));
  };

  f32x16 oacc[C::QB][C::MB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) oacc[qb][mb] = f32x16{};
  float m_run[C::QB], l_run[C::QB];  // running max (log2 domain), lane's partial row sum
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  const float c = p.scale_log2;
  const bool causal = p.causal != 0;

  // one K/V tile; STAGE is compile-time so every LDS object and offset is fixed
  auto step = [&](auto stage, int t) {
    constexpr int ST = decltype(stage)::value;
    using Ahead = std::integral_constant<int, (ST + C::NS - 1) % C::NS>;
    // tile t complete; the tiles after it that were issued stay in flight
    if (t + 2 < nt) wait_vmem_le<2 * C::VMEM>();
    else if (t + 1 < nt) wait_vmem_le<C::VMEM>();
    else wait_vmem_le<0>();
    barrier_only();  // tile t visible to all waves; stage of tile t-1 free
    if (t + 3 < nt) issue_tile(t + 3, Ahead{});
    const lds_char* kt = ktile(stage);
    const lds_char* vt = vtile(stage);
    const int* kp = ptile(stage) + wave * C::BN;
    const int kfirst = uniform(kp[0]);
    const int klast = uniform(kp[C::BN - 1]);
    const int valid = min(C::BN, p.sk - (tb + t) * C::BN);
    const bool tail = valid < C::BN;
    if (!wave_live || (causal && kfirst > wqmax) || klast < wqs_min) return;

    f32x16 s[C::QB][C::NKB];
    // The two 32-key halves alternate, and the scheduling groups below keep
    // each K operand's LDS read four MFMAs ahead of its use (four reads, then
    // one after every MFMA).  Without them the first half's reads sat right
    // before their MFMAs, each waiting out the LDS latency.
    auto scores = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
          const bf16x8 a = lds_read_b128(kt, kb * 32 * D * 2 + koff[ks]);
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb)
            s[qb][kb] = mfma32x32x16(a, qf[qb][ks], ks == 0 ? f32x16{} : s[qb][kb]);
        }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < C::KS * C::NKB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };
    scores();

    uint32_t pk[C::QB][C::NKB][8];
    auto exps = [&](int qb, float neg_m, float& ps0, float& ps1) __attribute__((always_inline)) {
      ps0 = 0.f;
      ps1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float e0 = fast_exp2(fmaf(s[qb][kb][i], c, neg_m));
          const float e1 = fast_exp2(fmaf(s[qb][kb][i + 1], c, neg_m));
          pk[qb][kb][i >> 1] = pack_bf16x2(e0, e1);
          if (i & 2) ps1 += e0 + e1; else ps0 += e0 + e1;
        }
    };
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      // straddles this block's positions or sample starts
      const bool straddle = tail || (causal && klast > bmin[qb]) || kfirst < bqs_max[qb];
      // Unmasked tile of rows that all have a running max: exponentiate against
      // it directly.  A weight above 2^16 (a row max more than 16 above the
      // running one) sends the tile down the path that finds the tile max
      // and rescales, after recomputing the scores the exponentials used up.
      bool slow = straddle || __ballot(m_run[qb] == -INFINITY) != 0;
      float ps0 = 0.f, ps1 = 0.f;
      if (!slow) {
        exps(qb, -m_run[qb], ps0, ps1);
        if (__ballot(!(ps0 + ps1 <= 65536.0f))) {
          asm volatile("" ::: "memory");
          slow = true;
          scores();
        }
      }
      if (slow) {
        asm volatile("" ::: "memory");
        if (straddle) {
          // visible iff lo <= k_pos <= hi: one unsigned compare of k_pos - lo
          // against hi - lo (lo = the row's sample start, INT_MIN unless
          // packed; hi = its position, INT_MAX without the causal mask)
          const uint32_t lo = (uint32_t)qs[qb];
          const uint32_t span = (uint32_t)(causal ? qpos[qb] : INT_MAX) - lo;
          if (tail) {  // key slots past the chunk read position 0: drop them too
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
                const bool hide = ((uint32_t)kp[key] - lo > span) | (key >= valid);
                s[qb][kb][i] = hide ? -INFINITY : s[qb][kb][i];
              }
          } else {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
                s[qb][kb][i] = ((uint32_t)kp[key] - lo > span) ? -INFINITY : s[qb][kb][i];
              }
          }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[qb][kb][i]);
        mt = max_halves(mt) * c;
        if (__ballot(mt > m_run[qb] + 8.0f)) {
          asm volatile("" ::: "memory");
          const float m_new = fmaxf(m_run[qb], mt);
          const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[qb] - m_new);
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) oacc[qb][mb] *= alpha;
          l_run[qb] *= alpha;
          m_run[qb] = m_new;
        }
        exps(qb, (m_run[qb] == -INFINITY) ? 0.f : -m_run[qb], ps0, ps1);
      }
      l_run[qb] += ps0 + ps1;
    }

#pragma unroll
    for (int ks2 = 0; ks2 < C::BN / 16; ++ks2) {
      const int kb = ks2 >> 1, half = ks2 & 1;
      const int rb = ks2 * 16 * D * 2;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const bf16x8 a = lds_read_tr(vt, rb + voff[0][mb], rb + voff[1][mb]);
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) {
          const u32x4 bw = {pk[qb][kb][4 * half], pk[qb][kb][4 * half + 1],
                            pk[qb][kb][4 * half + 2], pk[qb][kb][4 * half + 3]};
          oacc[qb][mb] = mfma32x32x16(a, __builtin_bit_cast(bf16x8, bw), oacc[qb][mb]);
        }
      }
    }
  };

  if (nt > 0) issue_tile(0, S0{});
  if (nt > 1) issue_tile(1, S1{});
  if (nt > 2) issue_tile(2, S2{});
  for (int t = 0; t < nt; t += 4) {
    step(S0{}, t);
    if (t + 1 < nt) step(S1{}, t + 1);
    if (t + 2 < nt) step(S2{}, t + 2);
    if (t + 3 < nt) step(S3{}, t + 3);
  }

  // ---- epilogue: normalise, then write or merge ----
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const float l_tot = sum_halves(l_run[qb]);
    if (!row_ok[qb]) continue;
    const bool has = l_tot > 0.f;
    const float inv = has ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
    const float lse2 = has ? m_run[qb] + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    float* orow = p.o + ((size_t)row[qb] * p.hq + h) * D;
    float* lrow = p.lse + (size_t)h * p.sq + row[qb];
    if (!ACC) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = mb * 32 + 8 * g + 4 * hh;
          f32x4 val = {oacc[qb][mb][4 * g] * inv, oacc[qb][mb][4 * g + 1] * inv,
                       oacc[qb][mb][4 * g + 2] * inv, oacc[qb][mb][4 * g + 3] * inv};
          *(f32x4*)(orow + d0) = val;
        }
      if (hh == 0) *lrow = has ? lse2 * kLn2 : -INFINITY;
    } else {
      if (!has) continue;  // merging with an empty result is the identity
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
          for (int e = 0; e < 4; ++e) val[e] = fmaf(wa, old[e], wb * oacc[qb][mb][4 * g + e]);
          *(f32x4*)(orow + d0) = val;
        }
      if (hh == 0) *lrow = (mx + __builtin_amdgcn_logf(tot)) * kLn2;
    }
  }
}


template <int D>
hipError_t launch_fwd_d(const FwdParams& p, hipStream_t stream) {
  const dim3 grid(p.n_qtiles * p.hq), block(FwdCfg<D>::THREADS);
  // packed samples get their own instances so the plain causal path carries
  // no sample-start loads, compares or bounds
  const bool packed = p.q_start != nullptr;
  if (p.accumulate && packed)
    hipLaunchKernelGGL((attn_fwd_kernel<D, true, true>), grid, block, 0, stream, p);
  else if (p.accumulate)
    hipLaunchKernelGGL((attn_fwd_kernel<D, true, false>), grid, block, 0, stream, p);
  else if (packed)
    hipLaunchKernelGGL((attn_fwd_kernel<D, false, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, false, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int fwd_rows_per_block() { return FwdCfg<128>::BM; }

hipError_t launch_attn_fwd(const FwdParams& p, int d, hipStream_t stream) {
  return d == 64 ? launch_fwd_d<64>(p, stream) : launch_fwd_d<128>(p, stream);
}

}  // namespace mmsp
