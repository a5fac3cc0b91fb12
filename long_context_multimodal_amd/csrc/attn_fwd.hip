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
//    LDS ring with 16-byte direct loads (no staging registers); each stage
//    is one LDS object holding the K tile, the V tile and the tile's key
//    positions (one slot per wave), so the compiler tracks the loads into
//    one stage apart from reads of the others; rows past the chunk's end
//    lie outside the load's buffer range and arrive as zeros;
//  * the two waves on a SIMD (waves w and w + 4) run half a tile apart:
//    group 1 (waves 4-7) runs the same program one barrier behind group 0,
//    so while one wave runs its contractions (P V of tile t, then the
//    scores of tile t + 1, 32 MFMAs) the other runs the softmax of its
//    tile, and the matrix core and the vector ALU work at the same time.
//    The contracting wave raises its priority so the softmax beside it does
//    not hold back its MFMA issue.  Loads run two tiles ahead (a stage is
//    free once both groups finished P V of its tile);
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
//    tile back through the max-and-rescale path (the scores are still in
//    registers; the packed path recomputes them from the K tile in LDS);
//    row sums stay in fp32 (exact LSE for the merge and the backward);
//  * causal tile skipping from the sorted positions: a wave-wide search bounds
//    the key range of the workgroup, each wave skips tiles it cannot see and
//    masks only the tiles that straddle its rows' positions (or the tail),
//    with one unsigned compare per score (sample start <= key position <=
//    query position);
//  * packed samples (reset masks between samples packed in one buffer) take
//    a per-query sample start that also bounds the key range from below;
//    they run in their own template instance, so the plain path has none of
//    that code.  There all 8 waves step through the tiles together, three
//    tiles in flight, and a wave whose rows belong to other samples skips
//    the tile's contractions;
//  * GQA: query head h reads KV head h / G; the workgroup order keeps the
//    query heads of one KV head on one XCD (shared L2) and dispatches the
//    heavier (causally longer) query tiles first; when one head's tiles span
//    several XCDs, heavy and light tiles alternate in blocks of 8 so every
//    XCD and shader engine gets an even share;
//  * epilogue (plain instances): each wave passes its 32 rows of fp32 O
//    through the free K/V ring and reads O_acc and writes O in whole rows,
//    with the running result's reads issued before the loop's closing
//    barrier; packed instances store their 16-byte pieces directly.
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
  // one LDS object per pipeline stage: K tile, V tile, then the key
  // positions of the tile (one 64-entry slot per wave)
  static_assert(C::NS == 4, "stage objects below are written out for four stages");
  constexpr int STAGE = 2 * C::TILE + C::WAVES * C::BN * 4;
  __shared__ __attribute__((aligned(16))) char sS0[STAGE], sS1[STAGE], sS2[STAGE], sS3[STAGE];
  auto stage_base = [&](auto b) -> lds_char* {
    constexpr int S = decltype(b)::value;
    if constexpr (S == 0) return (lds_char*)sS0;
    else if constexpr (S == 1) return (lds_char*)sS1;
    else if constexpr (S == 2) return (lds_char*)sS2;
    else return (lds_char*)sS3;
  };
  auto ktile = [&](auto b) -> lds_char* { return stage_base(b); };
  auto vtile = [&](auto b) -> lds_char* { return stage_base(b) + C::TILE; };
  auto ptile = [&](auto b) -> int* { return (int*)(stage_base(b) + 2 * C::TILE); };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  int h = logical / p.n_qtiles;
  int qt = heavy_first_tile(logical % p.n_qtiles, p.n_qtiles, gridDim.x);
  // packed samples: tiles heaviest first from the plan, when one is given
  if (PACKED && plan_fits(p.plan, kPlanMagic, p.sq, p.sk))
    planned_tile(blockIdx.x, p.n_qtiles, p.hq, p.plan + p.plan_off, h, qt);
  const int kvh = h / p.group;
  const int q0 = qt * C::BM;
  const int wr0 = q0 + wave * 32 * C::QB;  // first row of this wave

  // ---- positions: per lane and block, per block range, workgroup range ----
  // Every position and sample start the prologue needs is read in one group
  // (indices clamped into the shard, results discarded where out of range),
  // so the reads overlap instead of waiting on one another.
  constexpr bool packed = PACKED;  // q_start given (keys below a row's sample start are hidden)
  const int sq1 = p.sq - 1;
  int row[C::QB], qpos[C::QB], bmin[C::QB], qs[C::QB], bqs_max[C::QB];
  bool row_ok[C::QB];
  int v_row[C::QB], v_r0[C::QB], v_qs[C::QB], v_bqs[C::QB];
  int v_wend = kPosInf - 1, v_qend = kPosInf - 1, v_wqs = INT_MIN, v_q0s = INT_MIN;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    row[qb] = wr0 + 32 * qb + l32;
    row_ok[qb] = row[qb] < p.sq;
    v_row[qb] = v_r0[qb] = kPosInf - 1;
    v_qs[qb] = v_bqs[qb] = INT_MIN;
  }
  if (p.causal) {
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      v_row[qb] = p.q_pos[min(row[qb], sq1)];
      v_r0[qb] = p.q_pos[min(wr0 + 32 * qb, sq1)];
    }
    v_wend = p.q_pos[min(wr0 + 32 * C::QB - 1, sq1)];
    v_qend = p.q_pos[min(q0 + C::BM - 1, sq1)];
  }
  if constexpr (packed) {
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      v_qs[qb] = p.q_start[min(row[qb], sq1)];
      v_bqs[qb] = p.q_start[min(wr0 + 32 * qb + 31, sq1)];
    }
    v_wqs = p.q_start[min(wr0, sq1)];
    v_q0s = p.q_start[min(q0, sq1)];
  }
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int r0 = wr0 + 32 * qb;
    qpos[qb] = row_ok[qb] ? v_row[qb] : INT_MIN;
    bmin[qb] = uniform(r0 < p.sq ? v_r0[qb] : kPosInf);
    qs[qb] = row_ok[qb] ? v_qs[qb] : INT_MIN;
    bqs_max[qb] = uniform(r0 < p.sq ? v_bqs[qb] : INT_MIN);
  }
  const bool wave_live = wr0 < p.sq;
  const int wqmax = uniform(wave_live ? v_wend : INT_MIN);
  const int wqs_min = uniform(wave_live ? v_wqs : INT_MIN);
  // key range of the workgroup: [kbeg, nk) -- keys at or below its last
  // position and, with packed samples, at or after its first sample start
  int nk = p.sk, kbeg = 0;
  if (p.causal) {
    if constexpr (packed)
      wave_prefix_two<true, false>(p.k_pos, p.sk, v_qend, p.k_pos, p.sk, v_q0s, nk, kbeg);
    else
      nk = wave_prefix<true>(p.k_pos, p.sk, v_qend);
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
  auto issue_tile = [&](int t, auto stage, bool live) {
    const int j0 = (tb + t) * C::BN;
    const size_t o = (size_t)j0 * kv_row_stride;
    const int rows = uniform(live ? min(C::BN, p.sk - j0) : 0);
    ld.load_rows(ktile(stage), kbase + o, rows);
    ld.load_rows(vtile(stage), vbase + o, rows);
    pos_load_direct((lds_char*)(ptile(stage) + wave * C::BN), pos_src, j0, rows);
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
    const lds_char* kt = ktile(stage);
    const lds_char* vt = vtile(stage);
    const int* kp = ptile(stage) + wave * C::BN;
    const int kfirst = uniform(kp[0]);
    const int klast = uniform(kp[C::BN - 1]);
    const int valid = min(C::BN, p.sk - (tb + t) * C::BN);
    const bool tail = valid < C::BN;
    // A wave whose rows cannot see the tile takes the masked path (all keys
    // hidden, zero weights) instead of a branch, so that the next tiles'
    // loads and the contractions below share one scheduling region.  Packed
    // samples are the exception: there whole waves often belong to another
    // sample than the tile, and skipping leaves the matrix core to the other
    // wave on the SIMD, so they issue the loads first and leave the step.
    const bool blind = !wave_live || (causal && kfirst > wqmax) || klast < wqs_min;
    if constexpr (PACKED) {
      issue_tile(t + 3, Ahead{}, t + 3 < nt);
      if (blind) return;
    }

    f32x16 s[C::QB][C::NKB];
    // The two 32-key halves alternate, and the scheduling groups below keep
    // each K operand's LDS read four MFMAs ahead of its use (four reads, then
    // one after every MFMA).  Without them the first half's reads sat right
    // before their MFMAs, each waiting out the LDS latency.
    auto scores = [&](bool with_loads) __attribute__((always_inline)) {
      if (with_loads) issue_tile(t + 3, Ahead{}, t + 3 < nt);
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
        if (with_loads && (i & 1) && i < 2 * C::VMEM)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    };
    scores(!PACKED);

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
      const bool straddle =
          blind || tail || (causal && klast > bmin[qb]) || kfirst < bqs_max[qb];
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
          scores(false);
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

  if constexpr (PACKED) {
    if (nt > 0) issue_tile(0, S0{}, true);
    issue_tile(1, S1{}, nt > 1);
    issue_tile(2, S2{}, nt > 2);
    for (int t = 0; t < nt; t += 4) {
      step(S0{}, t);
      if (t + 1 < nt) step(S1{}, t + 1);
      if (t + 2 < nt) step(S2{}, t + 2);
      if (t + 3 < nt) step(S3{}, t + 3);
    }
  } else if (nt > 0) {
    // ---- two wave groups half a tile apart ----
    // Waves w and w + 4 share a SIMD.  Group 1 (waves 4-7) runs the same
    // program one barrier behind group 0, so while one group's waves run
    // their contractions (P V of tile t, then the scores of tile t + 1) the
    // other group's waves on the same SIMDs run the softmax of their tile.
    static_assert(C::QB == 1, "one 32-row block per wave");
    const int grp = uniform(wave >> 2);
    f32x16 s[C::NKB];
    uint32_t pk[C::NKB][8];
    // P V of the tile in stage SP, then the scores of tile ts (stage SS) with
    // the loads of tile ts + 2 among them (its stage, (SS + 2) % 4, held tile
    // ts - 2, whose P V both groups have finished).  Each operand is read two
    // MFMAs ahead of its use; the first two V^T operands (vpre) were read
    // before the barrier that starts the phase.
    auto pv_then_s = [&](auto sp, auto ss, int ts, const bf16x8 (&vpre)[2])
        __attribute__((always_inline)) {
      constexpr int SS = decltype(ss)::value;
      using Ahead2 = std::integral_constant<int, (SS + 2) % C::NS>;
      const lds_char* vt = vtile(sp);
      const lds_char* kt = ktile(ss);
      constexpr int NPV = C::BN / 16 * C::MB, NSC = C::KS * C::NKB;
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int ks2 = i / C::MB, mb = i % C::MB;
        const int kb = ks2 >> 1, half = ks2 & 1;
        const int rb = ks2 * 16 * D * 2;
        const bf16x8 a = i < 2 ? vpre[i] : lds_read_tr(vt, rb + voff[0][mb], rb + voff[1][mb]);
        const u32x4 bw = {pk[kb][4 * half], pk[kb][4 * half + 1], pk[kb][4 * half + 2],
                          pk[kb][4 * half + 3]};
        oacc[0][mb] = mfma32x32x16(a, __builtin_bit_cast(bf16x8, bw), oacc[0][mb]);
      }
      issue_tile(ts + 2, Ahead2{}, ts + 2 < nt);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
          const bf16x8 a = lds_read_b128(kt, kb * 32 * D * 2 + koff[ks]);
          s[kb] = mfma32x32x16(a, qf[0][ks], ks == 0 ? f32x16{} : s[kb]);
        }
      // after MFMA i, the reads of MFMA i + 2 (two transposing reads for P V,
      // one b128 read for the scores); the loads among the scores
#pragma unroll
      for (int i = 0; i < NPV + NSC; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        const int j = i + 2;
        if (j < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else if (j < NPV + NSC) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (i >= NPV && ((i - NPV) & 1) && (i - NPV) < 2 * C::VMEM)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    };
    // the first tile's scores (and the loads of tile 2)
    auto s_only = [&](auto ss, int ts) __attribute__((always_inline)) {
      constexpr int SS = decltype(ss)::value;
      using Ahead2 = std::integral_constant<int, (SS + 2) % C::NS>;
      const lds_char* kt = ktile(ss);
      issue_tile(ts + 2, Ahead2{}, ts + 2 < nt);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
          const bf16x8 a = lds_read_b128(kt, kb * 32 * D * 2 + koff[ks]);
          s[kb] = mfma32x32x16(a, qf[0][ks], ks == 0 ? f32x16{} : s[kb]);
        }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < C::KS * C::NKB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + 2 < C::KS * C::NKB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if ((i & 1) && i < 2 * C::VMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    };
    // softmax of tile t (stage ST): masks, running max, exponentials -> pk,
    // row sums; the scores stay in registers for the max-and-rescale path
    auto softmax = [&](auto st, int t) __attribute__((always_inline)) {
      const int* kp = ptile(st) + wave * C::BN;
      const int kfirst = uniform(kp[0]);
      const int klast = uniform(kp[C::BN - 1]);
      const int valid = min(C::BN, p.sk - (tb + t) * C::BN);
      const bool tail = valid < C::BN;
      const bool blind = !wave_live || (causal && kfirst > wqmax);
      const bool straddle = blind || tail || (causal && klast > bmin[0]);
      auto exps = [&](float neg_m, float& ps0, float& ps1) __attribute__((always_inline)) {
        ps0 = 0.f;
        ps1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const float e0 = fast_exp2(fmaf(s[kb][i], c, neg_m));
            const float e1 = fast_exp2(fmaf(s[kb][i + 1], c, neg_m));
            pk[kb][i >> 1] = pack_bf16x2(e0, e1);
            if (i & 2) ps1 += e0 + e1; else ps0 += e0 + e1;
          }
      };
      bool slow = straddle || __ballot(m_run[0] == -INFINITY) != 0;
      float ps0 = 0.f, ps1 = 0.f;
      if (!slow) {
        exps(-m_run[0], ps0, ps1);
        slow = __ballot(!(ps0 + ps1 <= 65536.0f)) != 0;
      }
      if (slow) {
        asm volatile("" ::: "memory");
        if (straddle) {
          const uint32_t lo = (uint32_t)qs[0];
          const uint32_t span = (uint32_t)(causal ? qpos[0] : INT_MAX) - lo;
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
              const bool hide = ((uint32_t)kp[key] - lo > span) | (key >= valid) | blind;
              s[kb][i] = hide ? -INFINITY : s[kb][i];
            }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
        mt = max_halves(mt) * c;
        if (__ballot(mt > m_run[0] + 8.0f)) {
          asm volatile("" ::: "memory");
          const float m_new = fmaxf(m_run[0], mt);
          const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[0] - m_new);
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb) oacc[0][mb] *= alpha;
          l_run[0] *= alpha;
          m_run[0] = m_new;
        }
        exps((m_run[0] == -INFINITY) ? 0.f : -m_run[0], ps0, ps1);
      }
      l_run[0] += ps0 + ps1;
    };
    // One tile: [wait, barrier] softmax(t) [wait, barrier] P V(t) + S(t+1).
    // Tile t + 1 must be in LDS before group 0 starts its scores; every wave
    // waits for its share of it at both barriers (the loads of one later tile
    // stay in flight).  The wave running its contractions raises its priority
    // so that the softmax of the other wave on its SIMD (an older wave in
    // group 0) does not hold back its MFMA issue.
    auto tile = [&](auto st, auto sn, int t) __attribute__((always_inline)) {
      wait_vmcnt<C::VMEM>();
      barrier_only();
      softmax(st, t);
      bf16x8 vpre[2];
      {
        const lds_char* vt = vtile(st);
#pragma unroll
        for (int i = 0; i < 2; ++i) vpre[i] = lds_read_tr(vt, voff[0][i], voff[1][i]);
      }
      wait_vmcnt<C::VMEM>();
      barrier_only();
      // the last tile also runs the (unused) scores of tile nt: one code path
      __builtin_amdgcn_s_setprio(1);
      pv_then_s(st, sn, t + 1, vpre);
      __builtin_amdgcn_s_setprio(0);
    };
    issue_tile(0, S0{}, true);
    issue_tile(1, S1{}, nt > 1);
    wait_vmcnt<C::VMEM>();
    barrier_only();
    if (grp == 1) barrier_only();  // group 1 runs one barrier behind
    __builtin_amdgcn_s_setprio(1);
    s_only(S0{}, 0);
    __builtin_amdgcn_s_setprio(0);
    for (int t = 0; t < nt; t += 4) {
      tile(S0{}, S1{}, t);
      if (t + 1 < nt) tile(S1{}, S2{}, t + 1);
      if (t + 2 < nt) tile(S2{}, S3{}, t + 2);
      if (t + 3 < nt) tile(S3{}, S0{}, t + 3);
    }
    if (grp == 0) barrier_only();  // same barrier count in both groups
    wait_vmem_le<0>();
  }

  // ---- epilogue: normalise, then write or merge ----
  // A lane holds its row's head-dim entries in 16-byte pieces 32 bytes apart,
  // so storing them directly writes every fp32 row of O in 32-byte pieces, and
  // the workgroups of a plain causal launch end at about the same time, so
  // those pieces reach the L2 together.  Each wave instead passes its 32 rows through LDS
  // (the K/V ring is free after the loop) and reads and writes whole rows.
  // The pieces go in 1 KiB blocks, one per (32-column block, 8-row group);
  // lane L = 32 hh + r puts its piece in slot L ^ b ^ 8 hh of block b, so that
  // every 16-lane group of a dump or of a read-back touches 16 bank groups.
  static_assert(C::QB == 1, "one 32-row block per wave");
  if (ACC && nt == 0) {  // merging with an empty result is the identity
    wait_vmem_le<0>();
    return;
  }
  if constexpr (PACKED) {
    // Packed samples make many short workgroups that end at different times;
    // there the LDS pass costs more than the whole-row stores save (~5% of
    // the packed forward), so they store the 16-byte pieces directly.
    const float l_tot = sum_halves(l_run[0]);
    if (!row_ok[0]) return;
    const bool has = l_tot > 0.f;
    const float inv = has ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
    const float lse2 = has ? m_run[0] + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    float* orow = p.o + ((size_t)row[0] * p.hq + h) * D;
    float* lrow = p.lse + (size_t)h * p.sq + row[0];
    if (!ACC) {
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = mb * 32 + 8 * g + 4 * hh;
          f32x4 val = {oacc[0][mb][4 * g] * inv, oacc[0][mb][4 * g + 1] * inv,
                       oacc[0][mb][4 * g + 2] * inv, oacc[0][mb][4 * g + 3] * inv};
          *(f32x4*)(orow + d0) = val;
        }
      if (hh == 0) *lrow = has ? lse2 * kLn2 : -INFINITY;
    } else if (has) {  // merging with an empty result is the identity
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
          for (int e = 0; e < 4; ++e) val[e] = fmaf(wa, old[e], wb * oacc[0][mb][4 * g + e]);
          *(f32x4*)(orow + d0) = val;
        }
      if (hh == 0) *lrow = (mx + __builtin_amdgcn_logf(tot)) * kLn2;
    }
    return;
  }
  // The reads of the running result go out first, before the barrier: the
  // lane's row of LSE_acc, then every O_acc piece this lane merges below
  // (rows past sq read the last row and are not stored).
  constexpr int CH = D / 4;               // 16-byte pieces per fp32 row
  constexpr int READS = 32 * CH / kWave;  // pieces per lane
  const int cc = lane % CH;
  float la_raw = 0.f;
  f32x4 old[READS];
  if constexpr (ACC) {
    la_raw = p.lse[(size_t)h * p.sq + min(row[0], p.sq - 1)];
#pragma unroll
    for (int i = 0; i < READS; ++i) {
      const int r = min(wr0 + (i * kWave + lane) / CH, p.sq - 1);
      old[i] = *(const f32x4*)(p.o + ((size_t)r * p.hq + h) * D + cc * 4);
    }
  }
  wait_vmem_le<ACC ? READS + 1 : 0>();  // the direct loads into the ring have landed
  barrier_only();                       // and no wave reads the ring any more
  const float l_tot = sum_halves(l_run[0]);
  const bool has = l_tot > 0.f;
  const float inv = has ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
  const float lse2 = has ? m_run[0] + __builtin_amdgcn_logf(l_tot) : -INFINITY;
  // the lane's row: new O = wa * O_acc + wb * (unnormalised O of this chunk);
  // wa < 0 leaves the row as it is
  float wa = 0.f, wb = inv;
  if (row_ok[0]) {
    float* lrow = p.lse + (size_t)h * p.sq + row[0];
    if (!ACC) {
      if (hh == 0) *lrow = has ? lse2 * kLn2 : -INFINITY;
    } else if (!has) {
      wa = -1.f;  // merging with an empty result is the identity
    } else {
      const float la2 = la_raw * kLog2e;  // -inf stays -inf
      const float mx = fmaxf(la2, lse2);
      const float ea = fast_exp2(la2 - mx), eb = fast_exp2(lse2 - mx);
      const float tot = ea + eb;
      const float rt = __builtin_amdgcn_rcpf(tot);
      wa = ea * rt;
      wb = eb * rt * inv;
      if (hh == 0) *lrow = (mx + __builtin_amdgcn_logf(tot)) * kLn2;
    }
  }
  // waves 2s and 2s + 1 use stage s: one tile each for their 32 rows of fp32 O
  // (32 x D x 4 bytes = one K or V tile), their row factors in its position slots
  static_assert(32 * D * 4 == C::TILE && 2 * 32 * 4 <= C::WAVES * C::BN * 4,
                "two waves' rows and row factors fit one stage");
  const int w2 = wave >> 1;
  lds_char* stg = w2 == 0 ? (lds_char*)sS0 : w2 == 1 ? (lds_char*)sS1
                : w2 == 2 ? (lds_char*)sS2 : (lds_char*)sS3;
  lds_char* reg = stg + (wave & 1) * C::TILE;
  float* wa_s = (float*)(stg + 2 * C::TILE) + (wave & 1) * 32;
  if (ACC && hh == 0) wa_s[l32] = wa;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int b = mb * 4 + g;
      const f32x4 v4 = {oacc[0][mb][4 * g] * wb, oacc[0][mb][4 * g + 1] * wb,
                        oacc[0][mb][4 * g + 2] * wb, oacc[0][mb][4 * g + 3] * wb};
      *(__attribute__((address_space(3))) f32x4*)(reg + b * 1024 + ((lane ^ b ^ (hh << 3)) << 4)) =
          v4;
    }
  wait_lds_writes();
  // read back: step i covers rows rr = (64 i + lane) / CH, piece cc = lane % CH
  // (columns 4 cc .. 4 cc + 3), which sits in block cc / 2, lane slot
  // (cc % 2) * 32 + rr
  // (all pieces are read before the first store, so the reads overlap)
  const int rb = cc >> 1;
  const lds_char* rbase = reg + rb * 1024;
  f32x4 piece[READS];
  float a[READS];
#pragma unroll
  for (int i = 0; i < READS; ++i) {
    const int rr = (i * kWave + lane) / CH;
    const int slot = ((cc & 1) << 5) | rr;
    piece[i] = *(const __attribute__((address_space(3))) f32x4*)(
        rbase + ((slot ^ rb ^ ((cc & 1) << 3)) << 4));
    a[i] = ACC ? wa_s[rr] : 0.f;
  }
  wait_lds_writes();  // lgkmcnt(0): every read above has returned
#pragma unroll
  for (int i = 0; i < READS; ++i) {
    const int r = wr0 + (i * kWave + lane) / CH;
    f32x4 v4 = piece[i];
    if constexpr (ACC) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = fmaf(a[i], old[i][e], v4[e]);
    }
    if (r < p.sq && (!ACC || a[i] >= 0.f))
      *(f32x4*)(p.o + ((size_t)r * p.hq + h) * D + cc * 4) = v4;
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

static_assert(FwdCfg<64>::BM == FwdCfg<128>::BM && FwdCfg<64>::BN == FwdCfg<128>::BN,
              "tile plans are laid out for one tile shape per kernel");
int fwd_rows_per_block() { return FwdCfg<128>::BM; }
int fwd_keys_per_tile() { return FwdCfg<128>::BN; }

hipError_t launch_attn_fwd(const FwdParams& p, int d, hipStream_t stream) {
  return d == 64 ? launch_fwd_d<64>(p, stream) : launch_fwd_d<128>(p, stream);
}

}  // namespace mmsp
