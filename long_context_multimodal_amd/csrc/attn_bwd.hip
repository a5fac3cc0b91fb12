// Backward of causal attention of a query shard against one KV chunk (gfx950).
//
// The pages train at 2M tokens without gradient checkpointing ("LongVILA -
// ... (Jason's Study)", section "What it is"), so the backward consumes the
// forward's saved output and log-sum-exp: P = exp(scale q.k - LSE_final) on
// visible pairs, dV = P^T dO, dS = P o (dO V^T - delta), dQ += scale dS K,
// dK = scale dS^T Q, with dK/dV of a KV head summed over its query heads.
//
// Two kernels, no atomics:
//  * dK/dV kernel -- one workgroup = 128 keys of one KV head (4 waves of 32
//    keys).  K of the wave's keys stays in registers as the B operand of
//    S = Q K^T, the workgroup's V rows sit in LDS as the B operand of
//    dP = dO V^T, and the dK^T / dV^T accumulators stay in registers.  The
//    workgroup walks the visible query tiles (32 rows) of every query head
//    of its KV head; Q and dO tiles arrive by direct global->LDS loads into
//    swizzled double buffers and serve both as row-major A operands (S, dP)
//    and, through the transposing LDS read, as Q^T / dO^T (dK^T, dV^T),
//    whose B operands are the P / dS accumulators reused in place.
//  * dQ kernel -- one workgroup = 128 query rows of one query head (like the
//    forward): Q and dO stay in registers, K/V tiles stream through LDS,
//    S^T = K Q^T and dP^T = V dO^T give P^T and dS^T with the query in the
//    lane (so LSE and delta are per-lane scalars), and dQ^T += K^T dS^T uses
//    the transposing read of the K tile.  dQ is added to dq_acc once per
//    workgroup (plain read-modify-write: each element has one owner).
// Recomputing S and dP in the dQ kernel costs two extra contractions per
// visible pair; it replaces fp32 atomics, which on this part execute past
// the L2 and cost more than the recomputation.
//
// Causal skipping in both: the key (or query) range of a workgroup is
// bounded by a wave-wide search on the sorted positions, waves skip tiles they
// cannot see and mask only the tiles that straddle their positions.  Packed
// samples (a per-query sample start bounding the keys from below) run in
// their own template instances.  Either kernel can be enqueued alone
// (run_dkdv / run_dq), so a caller may put the two on separate streams.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mmsp {
namespace {

// ============================== dK / dV ======================================
template <int D>
struct DkdvCfg {
  static constexpr int BK = 128;          // keys per workgroup
  static constexpr int BQ = 32;           // queries per tile
  static constexpr int THREADS = 256;
  static constexpr int KS = D / 16;
  static constexpr int MB = D / 32;
  static constexpr int TILE = BQ * D * 2;  // bytes of one Q or dO tile
  static constexpr int VTILE = BK * D * 2; // bytes of the workgroup's V rows
};

template <int D, bool PACKED>
__global__ void __launch_bounds__(256, 2) attn_bwd_dkdv_kernel(BwdParams p) {
  using C = DkdvCfg<D>;
  // one LDS object per pipeline buffer (the compiler then knows the direct
  // loads into one buffer never alias reads of the other)
  __shared__ __attribute__((aligned(16))) char sQ0[C::TILE], sQ1[C::TILE];
  __shared__ __attribute__((aligned(16))) char sO0[C::TILE], sO1[C::TILE];
  __shared__ __attribute__((aligned(16))) char sVrows[C::VTILE];
  // per-row statistics of the two tiles in flight, one row of 36 words per
  // (statistic, buffer): 0 sample starts (packed), 1 -LSE/scale (-inf for
  // empty rows and rows past sq), 2 -delta, 3 positions (word 32: the tile's
  // last position).  Rows 1 and 2 are where the S and dP accumulators start,
  // so that exp2(c S) is the weight and dP arrives as dP - delta.
  constexpr int SROW = 36;
  __shared__ __attribute__((aligned(16))) uint32_t sStat[4][2][SROW];
  auto sQs = [&](int b) -> const int* { return (const int*)sStat[0][b]; };
  auto sL = [&](int b) -> const float* { return (const float*)sStat[1][b]; };
  auto sDl = [&](int b) -> const float* { return (const float*)sStat[2][b]; };
  auto sQp = [&](int b) -> const int* { return (const int*)sStat[3][b]; };
  auto qtile = [&](auto b) -> lds_char* {
    if constexpr (decltype(b)::value == 0) return (lds_char*)sQ0; else return (lds_char*)sQ1;
  };
  auto otile = [&](auto b) -> lds_char* {
    if constexpr (decltype(b)::value == 0) return (lds_char*)sO0; else return (lds_char*)sO1;
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  int kvh = logical / p.n_ktiles;
  // early keys see more queries: their end of the range is dispatched first
  int kt = p.n_ktiles - 1 - heavy_first_tile(logical % p.n_ktiles, p.n_ktiles, gridDim.x);
  // packed samples: tiles heaviest first from the plan, when one is given
  if (PACKED && plan_fits(p.plan, kPlanMagic, p.sq, p.sk))
    planned_tile(blockIdx.x, p.n_ktiles, p.hkv, p.plan + p.plan_dkdv_off, kvh, kt);
  const int j0 = kt * C::BK;
  const int key = j0 + wave * 32 + l32;
  const bool key_ok = key < p.sk;
  const size_t kv_stride = (size_t)p.hkv * D;

  // Every key position the prologue needs is read in one group (indices
  // clamped into the chunk), so the reads overlap instead of waiting on one
  // another; then one wave-wide search finds the visible query range.
  const int sk1 = p.sk - 1;
  const int wk0 = j0 + wave * 32;
  const bool wave_live = wk0 < p.sk;
  const bool wave_full_keys = wk0 + 31 < p.sk;
  int v_key = 0, v_w0 = 0, v_wend = 0, v_j0 = 0, v_jend = 0;
  if (p.causal) {
    v_key = p.k_pos[min(key, sk1)];
    v_w0 = p.k_pos[min(wk0, sk1)];
    v_wend = p.k_pos[min(wk0 + 31, sk1)];
    v_j0 = p.k_pos[j0];
    v_jend = p.k_pos[min(j0 + C::BK - 1, sk1)];
  }
  const int kpos = key_ok ? v_key : kPosInf;
  const int wkmin = uniform(wave_live ? v_w0 : kPosInf);
  const int wkmax = uniform(wave_live ? v_wend : kPosInf);
  // queries at or after the workgroup's first key position and, with packed
  // samples, whose sample starts at or before its last key (sample starts
  // are non-decreasing): both ends from one wave-wide search
  constexpr bool packed = PACKED;  // q_start given
  int qstart = 0, qend = p.sq;
  if (p.causal) {
    if constexpr (packed)
      wave_prefix_two<false, true>(p.q_pos, p.sq, v_j0, p.q_start, p.sq, v_jend, qstart, qend);
    else
      qstart = wave_prefix<false>(p.q_pos, p.sq, v_j0);
  }
  const int n_qt = uniform((qend + C::BQ - 1) / C::BQ);
  const int qt0 = qstart / C::BQ;
  const int per_head = n_qt - qt0;
  const int total = uniform(per_head > 0 ? per_head * p.group : 0);

  // stationary K fragments (B operand of S: col = key, k = head dim); the
  // workgroup's V rows go to LDS once (B operand of dP, read like Q rows)
  bf16x8 kf[C::KS];
  {
    const uint16_t* kr = p.k + (size_t)key * kv_stride + (size_t)kvh * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u};
      if (key_ok) a = *(const u32x4*)(kr + 16 * ks);
      kf[ks] = __builtin_bit_cast(bf16x8, a);
    }
    TileLoader<D, C::BK, C::THREADS> vld;
    vld.init(tid, kv_stride);
    const uint16_t* vb = p.v + (size_t)j0 * kv_stride + (size_t)kvh * D;
    if (j0 + C::BK <= p.sk) vld.load((lds_char*)sVrows, vb);
    else vld.load_clamped((lds_char*)sVrows, vb, kv_stride, p.sk - j0);
  }
  const lds_char* vrows = (lds_char*)sVrows + uniform(wave * 32 * D * 2);

  int qoff[C::KS];  // A = Q / dO rows: row l32, chunk 2 ks + hh
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) qoff[ks] = tile_off<D>(l32, 2 * ks + hh);
  int troff[2][C::MB];  // A = Q^T / dO^T: rows 16 ks + ..., cols 32 mb + l32
#pragma unroll
  for (int rh = 0; rh < 2; ++rh)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) troff[rh][mb] = tr_offset<D>(lane, 0, rh, mb);

  const size_t q_row_stride = (size_t)p.hq * D;
  TileLoader<D, C::BQ, C::THREADS> ld;
  ld.init(tid, q_row_stride);
  uint32_t stat = 0;
  bool row_live = false;

  // Tiles in order: query heads kvh*G .. kvh*G+G-1, each over query tiles
  // qt0 .. n_qt-1.  Tiles are fetched in sequence, so the next one is tracked
  // by counters rather than recomputed with divisions.
  int nx_h = kvh * p.group, nx_q0 = qt0 * C::BQ;
  // Running element offset of the next tile's first Q / dO element: one row
  // block further per tile, one head further (and back to qt0) per head.
  const size_t tile_step = (size_t)C::BQ * q_row_stride;
  size_t nx_off = (size_t)nx_q0 * q_row_stride + (size_t)nx_h * D;
  const size_t head_back = (size_t)(n_qt - qt0) * tile_step - D;
  // Per-row statistics, one array per wave (0: sample starts when packed,
  // 1: LSE, 2: delta, 3: positions, its lane BQ fetching the tile's last
  // position), all into the one register `stat`; the array and its per-head
  // stride are fixed per wave before the loop.
  const uint32_t* stat_src = (wave == 0 && packed) ? (const uint32_t*)p.q_start
                             : wave == 2           ? (const uint32_t*)p.delta
                             : (wave == 3 && p.causal) ? (const uint32_t*)p.q_pos
                                                   : (const uint32_t*)p.lse;  // any readable row
  const size_t stat_head = (wave == 1 || wave == 2) ? (size_t)p.sq : 0;
  // Loads of the next tile, without branches, so that the scheduler can
  // spread them between the contractions of the current one (issued all at
  // once they queue behind the other waves' at the texture unit).  With no
  // next tile (`live` false) the buffer ranges are empty: the loads fetch
  // nothing and fill the unused buffer with zeros.
  auto issue_next = [&](auto buf, bool live) {
    const int h = min(nx_h, p.hq - 1), q0 = nx_q0;
    const size_t o = nx_off;
    const bool wrap = nx_q0 + C::BQ >= n_qt * C::BQ;
    nx_q0 = wrap ? qt0 * C::BQ : nx_q0 + C::BQ;
    nx_h = wrap ? nx_h + 1 : nx_h;
    nx_off = wrap ? nx_off + tile_step - head_back : nx_off + tile_step;
    // Raw statistics only: they are converted when published, after the wait
    // that ends the step, so no load here is waited for inside the step.
    const int i = min(q0 + min(lane, C::BQ - 1), p.sq - 1);
    if constexpr (packed) {
      // packed samples issue these at the top of the step (many short
      // workgroups), where the plain branches cost less than the clamped forms
      if (!live) return;
      if (q0 + C::BQ <= p.sq) {
        ld.load(qtile(buf), p.q + o);
        ld.load(otile(buf), p.dout + o);
      } else {
        ld.load_clamped(qtile(buf), p.q + o, q_row_stride, p.sq - q0);
        ld.load_clamped(otile(buf), p.dout + o, q_row_stride, p.sq - q0);
      }
      if (lane <= C::BQ) {
        stat = stat_src[(size_t)h * stat_head + i];
        row_live = q0 + lane < p.sq;
      }
    } else {
      const int rows = uniform(live ? min(C::BQ, p.sq - q0) : 0);
      ld.load_clamped(qtile(buf), p.q + o, q_row_stride, rows);
      ld.load_clamped(otile(buf), p.dout + o, q_row_stride, rows);
      stat = stat_src[(size_t)h * stat_head + i];
      row_live = q0 + lane < p.sq;
    }
  };
  // Each wave converts its statistic and writes it with one store: the
  // destination row is fixed per wave, so only the lane offset is a register.
  const float inv_scale = 1.0f / p.scale;
  auto publish_tile = [&](int buf) {
    if (lane <= C::BQ && (wave == 3 || lane < C::BQ)) {
      uint32_t val;
      if (wave == 0) {
        val = (packed && row_live) ? stat : (uint32_t)INT_MIN;
      } else if (wave == 1) {
        // -LSE / scale, the start of the S accumulator, so that c S' = c S -
        // LSE log2(e); empty rows and rows past sq get -inf (weights 0)
        const float l = __uint_as_float(stat);
        val = __float_as_uint((row_live && l != -INFINITY) ? -l * inv_scale : -INFINITY);
      } else if (wave == 2) {
        val = row_live ? (stat ^ 0x80000000u) : 0u;  // -delta, the start of dP
      } else {
        const int pos = p.causal ? (int)stat : kPosInf - 1;
        val = (uint32_t)((row_live || lane == C::BQ) ? pos : INT_MIN);
      }
      sStat[wave][buf][lane] = val;
    }
  };

  f32x16 dkacc[C::MB], dvacc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    dkacc[mb] = f32x16{};
    dvacc[mb] = f32x16{};
  }
  const float c = p.scale_log2;

  auto step = [&](auto buf_tag, int it) {
    constexpr int BUF = decltype(buf_tag)::value;
    using Next = std::integral_constant<int, BUF ^ 1>;
    const bool more = it + 1 < total;
    const lds_char* qt = qtile(buf_tag);
    const lds_char* dt = otile(buf_tag);
    const int qfirst = uniform(sQp(BUF)[0]);
    const int qlast = uniform(sQp(BUF)[C::BQ]);
    const int qs_first = packed ? uniform(sQs(BUF)[0]) : INT_MIN;
    const int qs_last = packed ? uniform(sQs(BUF)[C::BQ - 1]) : INT_MIN;
    // Every wave runs every tile: one whose keys the tile's rows cannot see
    // (only next to the causal diagonal) masks all its scores and adds zeros.
    // Without a branch here, the next tile's loads share one scheduling
    // region with the contractions below.  Packed samples issue the loads
    // first and skip such tiles: there a wave's keys often belong to another
    // sample than the tile's rows.
    const bool sees = wave_live && qlast >= wkmin && qs_first <= wkmax;
    if constexpr (packed) issue_next(Next{}, more);
    if (!packed || sees) {
      if constexpr (!packed) issue_next(Next{}, more);
      // S = Q K^T and dP = dO V^T  (row = query, col = key), accumulated onto
      // -LSE/scale and -delta of their rows
      f32x16 s0, d0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *(const f32x4*)&sL(BUF)[8 * g + 4 * hh];
        const f32x4 d4 = *(const f32x4*)&sDl(BUF)[8 * g + 4 * hh];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s0[4 * g + e] = l4[e];
          d0[4 * g + e] = d4[e];
        }
      }
      f32x16 s = mfma32x32x16(lds_read_b128(qt, qoff[0]), kf[0], s0);
      f32x16 dp = mfma32x32x16(lds_read_b128(dt, qoff[0]), lds_read_b128(vrows, qoff[0]), d0);
#pragma unroll
      for (int ks = 1; ks < C::KS; ++ks) {
        s = mfma32x32x16(lds_read_b128(qt, qoff[ks]), kf[ks], s);
        dp = mfma32x32x16(lds_read_b128(dt, qoff[ks]), lds_read_b128(vrows, qoff[ks]), dp);
      }
      // the next tile's loads spread between the contractions, one after
      // every other one, instead of queueing at the texture unit all at once
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      const int last_row_pos = uniform(sQp(BUF)[C::BQ - 1]);  // INT_MIN past sq
      // straddles the rows' positions or their sample starts (or the tail)
      if (!(wave_full_keys && qfirst >= wkmax && last_row_pos != INT_MIN && qs_last <= wkmin)) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = 8 * (i >> 2) + 4 * hh + (i & 3);
          bool hide = kpos > sQp(BUF)[q];
          if constexpr (packed) hide |= kpos < sQs(BUF)[q];
          s[i] = hide ? -INFINITY : s[i];
        }
      }
      uint32_t pk[8], dsk[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = fast_exp2(s[4 * g + e] * c);
          pv[e] = pe;
          dsv[e] = pe * dp[4 * g + e];
        }
        pk[2 * g] = pack_bf16x2(pv[0], pv[1]);
        pk[2 * g + 1] = pack_bf16x2(pv[2], pv[3]);
        dsk[2 * g] = pack_bf16x2(dsv[0], dsv[1]);
        dsk[2 * g + 1] = pack_bf16x2(dsv[2], dsv[3]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // dV^T += dO^T P and dK^T += Q^T dS  (row = head dim, col = key, k = query)
#pragma unroll
      for (int ks = 0; ks < C::BQ / 16; ++ks) {
        const u32x4 pw = {pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
        const u32x4 sw = {dsk[4 * ks], dsk[4 * ks + 1], dsk[4 * ks + 2], dsk[4 * ks + 3]};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        const bf16x8 sb = __builtin_bit_cast(bf16x8, sw);
        const int rb = ks * 16 * D * 2;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          dvacc[mb] = mfma32x32x16(lds_read_tr(dt, rb + troff[0][mb], rb + troff[1][mb]), pb,
                                   dvacc[mb]);
          dkacc[mb] = mfma32x32x16(lds_read_tr(qt, rb + troff[0][mb], rb + troff[1][mb]), sb,
                                   dkacc[mb]);
        }
      }
      // keep 8 transposing reads in flight ahead of the MFMA that consumes them
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    if (more) {
      publish_tile(BUF ^ 1);
      wait_vmem();
    }
    __syncthreads();
  };

  if (total > 0) {
    issue_next(B0{}, true);
    publish_tile(0);
  }
  wait_vmem();
  __syncthreads();
  for (int it = 0; it < total; it += 2) {
    step(B0{}, it);
    if (it + 1 < total) step(B1{}, it + 1);
  }

  // ---- epilogue: dK = scale * (dK^T)^T, dV = (dV^T)^T ----
  // A lane holds one key's head-dim entries in 16-byte pieces that sit 32
  // bytes apart, so storing them directly writes each row in 32-byte pieces.
  // Each wave instead passes its 32 keys through LDS (free after the loop's
  // last barrier) and writes whole rows: a store of 64 lanes x 16 bytes covers
  // 1 KiB of consecutive rows.  The accumulator's 16-byte pieces are dumped
  // as they are, one 1 KiB block b per (32-column block, 8-row group), lane
  // L = 32 hh + r's piece in slot L ^ b ^ 8 hh: each dump is a 1 KiB write
  // whose 16-lane groups cover 16 bank groups, and so are the 16-lane groups
  // that read back one row's pieces (blocks b = 0..7 of both halves hh).
  if (!wave_live) return;
  constexpr int NB = C::MB * 4;          // 1 KiB blocks per accumulator
  constexpr int CH = D / 4;              // 16-byte pieces per fp32 row
  constexpr int READS = 32 * CH / kWave; // pieces per lane
  static_assert(NB / 2 * 1024 <= C::TILE, "half the blocks fit one Q/dO tile buffer");
  lds_char* reg0;
  lds_char* reg1;  // blocks [0, NB/2) and [NB/2, NB) of this wave
  if (wave < 2) {
    reg0 = (lds_char*)sVrows + wave * NB * 1024;
    reg1 = reg0 + NB / 2 * 1024;
  } else if (wave == 2) {
    reg0 = (lds_char*)sQ0;
    reg1 = (lds_char*)sQ1;
  } else {
    reg0 = (lds_char*)sO0;
    reg1 = (lds_char*)sO1;
  }
  // the piece a lane reads in step i: row rr = (i * 64 + lane) / CH of the
  // wave's 32 keys, columns 4 cc .. 4 cc + 3, cc = lane % CH, which lives in
  // block b = cc / 2 (mb = b / 4, g = b % 4), lane slot (cc % 2) * 32 + rr
  const int cc = lane % CH;
  const int rb = cc >> 1;
  lds_char* rbase = (rb < NB / 2 ? reg0 + rb * 1024 : reg1 + (rb - NB / 2) * 1024);
  auto store_rows = [&](const f32x16* acc, float mul, float* out) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int b = mb * 4 + g;
        lds_char* blk = (b < NB / 2 ? reg0 + b * 1024 : reg1 + (b - NB / 2) * 1024);
        const f32x4 v4 = {acc[mb][4 * g] * mul, acc[mb][4 * g + 1] * mul,
                          acc[mb][4 * g + 2] * mul, acc[mb][4 * g + 3] * mul};
        *(__attribute__((address_space(3))) f32x4*)(blk + ((lane ^ b ^ (hh << 3)) << 4)) = v4;
      }
    wait_lds_writes();
    // the pieces are read (and, to accumulate, the old values loaded) eight
    // at a time before any of them is stored, so the reads overlap
    constexpr int GRP = READS < 8 ? READS : 8;
#pragma unroll
    for (int i0 = 0; i0 < READS; i0 += GRP) {
      f32x4 piece[GRP];
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const int rr = ((i0 + j) * kWave + lane) / CH;
        const int slot = ((cc & 1) << 5) | rr;
        piece[j] = *(const __attribute__((address_space(3))) f32x4*)(
            rbase + ((slot ^ rb ^ ((cc & 1) << 3)) << 4));
      }
      wait_lds_writes();  // lgkmcnt(0): every read above has returned
      if (p.accumulate) {
#pragma unroll
        for (int j = 0; j < GRP; ++j) {  // keys past sk read the last key and are not stored
          const int k = min(wk0 + ((i0 + j) * kWave + lane) / CH, p.sk - 1);
          piece[j] += *(const f32x4*)(out + (size_t)k * kv_stride + (size_t)kvh * D + cc * 4);
        }
      }
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const int k = wk0 + ((i0 + j) * kWave + lane) / CH;
        if (k < p.sk) *(f32x4*)(out + (size_t)k * kv_stride + (size_t)kvh * D + cc * 4) = piece[j];
      }
    }
  };
  store_rows(dkacc, p.scale, p.dk);
  wait_lds_writes();  // the reads of dK's pieces are done before dV's dump reuses the blocks
  store_rows(dvacc, 1.0f, p.dv);
}

// ================================== dQ =======================================
template <int D>
struct DqCfg {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int THREADS = 256;
  static constexpr int KS = D / 16;
  static constexpr int MB = D / 32;
  static constexpr int NKB = BN / 32;
  static constexpr int TILE = BN * D * 2;
};

template <int D, bool PACKED>
__global__ void __launch_bounds__(256, 2) attn_bwd_dq_kernel(BwdParams p) {
  using C = DqCfg<D>;
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
  int h = logical / p.n_qtiles;
  int qt = heavy_first_tile(logical % p.n_qtiles, p.n_qtiles, gridDim.x);
  // packed samples: tiles heaviest first from the plan, when one is given
  if (PACKED && plan_fits(p.plan, kPlanMagic, p.sq, p.sk))
    planned_tile(blockIdx.x, p.n_qtiles, p.hq, p.plan + p.plan_dq_off, h, qt);
  const int kvh = h / p.group;
  const int q0 = qt * C::BM;
  const int row = q0 + wave * 32 + l32;
  const bool row_ok = row < p.sq;

  // Every position, sample start and row statistic the prologue needs is
  // read in one group (indices clamped into the shard, results discarded
  // where out of range), so the reads overlap instead of waiting on one another.
  constexpr bool packed = PACKED;  // q_start given (keys below a row's sample start are hidden)
  const int sq1 = p.sq - 1;
  const int wr0 = q0 + wave * 32;
  const bool wave_live = wr0 < p.sq;
  const int rc = min(row, sq1);
  const float l_raw = p.lse[(size_t)h * p.sq + rc];
  const float d_raw = p.delta[(size_t)h * p.sq + rc];
  int v_row = kPosInf - 1, v_w0 = kPosInf - 1, v_wend = kPosInf - 1, v_qend = kPosInf - 1;
  if (p.causal) {
    v_row = p.q_pos[rc];
    v_w0 = p.q_pos[min(wr0, sq1)];
    v_wend = p.q_pos[min(wr0 + 31, sq1)];
    v_qend = p.q_pos[min(q0 + C::BM - 1, sq1)];
  }
  int v_qs = INT_MIN, v_wqs0 = INT_MIN, v_wqs1 = INT_MIN, v_q0s = INT_MIN;
  if constexpr (packed) {
    v_qs = p.q_start[rc];
    v_wqs0 = p.q_start[min(wr0, sq1)];
    v_wqs1 = p.q_start[min(wr0 + 31, sq1)];
    v_q0s = p.q_start[min(q0, sq1)];
  }
  const int qpos = row_ok ? v_row : INT_MIN;
  const float lse2 = !row_ok ? INFINITY : (l_raw == -INFINITY) ? INFINITY : l_raw * kLog2e;
  const float delta = row_ok ? d_raw : 0.f;
  const int wqmin = uniform(wave_live ? v_w0 : 0);
  const int wqmax = uniform(wave_live ? v_wend : INT_MIN);
  const int qs = row_ok ? v_qs : INT_MIN;
  const int wqs_min = uniform(wave_live ? v_wqs0 : INT_MIN);
  const int wqs_max = uniform(wave_live ? v_wqs1 : INT_MIN);
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

  // Q and dO fragments: B operands of S^T = K Q^T and dP^T = V dO^T
  bf16x8 qf[C::KS], df[C::KS];
  {
    const size_t ro = ((size_t)row * p.hq + h) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (row_ok) {
        a = *(const u32x4*)(p.q + ro + 16 * ks);
        b = *(const u32x4*)(p.dout + ro + 16 * ks);
      }
      qf[ks] = __builtin_bit_cast(bf16x8, a);
      df[ks] = __builtin_bit_cast(bf16x8, b);
    }
  }

  int koff[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) koff[ks] = tile_off<D>(l32, 2 * ks + hh);
  int troff[2][C::MB];
#pragma unroll
  for (int rh = 0; rh < 2; ++rh)
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) troff[rh][mb] = tr_offset<D>(lane, 0, rh, mb);

  const size_t kv_row_stride = (size_t)p.hkv * D;
  const uint16_t* kbase = p.k + (size_t)kvh * D;
  const uint16_t* vbase = p.v + (size_t)kvh * D;
  TileLoader<D, C::BN, C::THREADS> ld;
  ld.init(tid, kv_row_stride);
  int kpreg = kPosInf;
  bool key_live = false;
  // Loads of tile t without branches (see the dK/dV kernel): with `live`
  // false the ranges are empty and nothing is fetched.  Every thread reads a
  // position (clamped into the array); threads below BN publish theirs.
  auto issue_tile = [&](int t, auto buf, bool live) {
    const int j0 = (tb + t) * C::BN;
    const size_t o = (size_t)j0 * kv_row_stride;
    if constexpr (packed) {  // at the top of the step, plain branches (see dK/dV)
      if (!live) return;
      if (j0 + C::BN <= p.sk) {
        ld.load(ktile(buf), kbase + o);
        ld.load(vtile(buf), vbase + o);
      } else {
        ld.load_clamped(ktile(buf), kbase + o, kv_row_stride, p.sk - j0);
        ld.load_clamped(vtile(buf), vbase + o, kv_row_stride, p.sk - j0);
      }
      if (tid < C::BN) {  // raw position; keys past sk are hidden when published
        kpreg = p.causal ? p.k_pos[min(j0 + tid, p.sk - 1)] : 0;
        key_live = j0 + tid < p.sk;
      }
    } else {
      const int rows = uniform(live ? min(C::BN, p.sk - j0) : 0);
      ld.load_clamped(ktile(buf), kbase + o, kv_row_stride, rows);
      ld.load_clamped(vtile(buf), vbase + o, kv_row_stride, rows);
      // raw position; keys past sk are hidden when published
      kpreg = p.causal ? p.k_pos[max(0, min(j0 + (tid & (C::BN - 1)), p.sk - 1))] : 0;
      key_live = j0 + (tid & (C::BN - 1)) < p.sk;
    }
  };

  f32x16 dqacc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) dqacc[mb] = f32x16{};
  const float c = p.scale_log2;

  auto step = [&](auto buf_tag, int t) {
    constexpr int BUF = decltype(buf_tag)::value;
    using Next = std::integral_constant<int, BUF ^ 1>;
    const bool more = t + 1 < nt;
    const lds_char* kt = ktile(buf_tag);
    const lds_char* vt = vtile(buf_tag);
    const int* kp = kpos_of(buf_tag);
    const int kfirst = uniform(kp[0]);
    const int klast = uniform(kp[C::BN - 1]);
    // Every wave runs every tile: one whose rows cannot see it (only next to
    // the causal diagonal, or rows past sq) takes the masked path, which
    // hides all its keys, and adds zeros.  Packed samples issue the loads
    // first and skip such tiles (see the dK/dV kernel).
    const bool sees = wave_live && kfirst <= wqmax && klast >= wqs_min;
    if constexpr (packed) issue_tile(t + 1, Next{}, more);
    if (!packed || sees) {
      // straddles the rows' positions or their sample starts
      const bool straddle = !wave_live || klast > wqmin || kfirst < wqs_max;
      static_assert(C::NKB == 2, "two 32-key blocks per tile");
      constexpr int LA = 2;  // operand reads ahead of their contraction
      constexpr int EPM = 16 / C::KS;  // vector items per contraction
      f32x16 dinit;
#pragma unroll
      for (int i = 0; i < 16; ++i) dinit[i] = -delta;  // dP accumulates onto -delta
      // S of block kb (K operands read LA contractions ahead), with side(i)
      // after contraction i; a scheduling barrier after every group holds the
      // order
      auto scores = [&](int kb, auto side) {
        const int rb = kb * 32 * D * 2;
        bf16x8 op[C::KS];
#pragma unroll
        for (int i = 0; i < LA; ++i) op[i] = lds_read_b128(kt, rb + koff[i]);
        f32x16 sc = f32x16{};
#pragma unroll
        for (int i = 0; i < C::KS; ++i) {
          if (i + LA < C::KS) op[i + LA] = lds_read_b128(kt, rb + koff[i + LA]);
          sc = mfma32x32x16(op[i], qf[i], sc);
          side(i);
          __builtin_amdgcn_sched_barrier(0);
        }
        return sc;
      };
      auto mask = [&](int kb, f32x16& sc) {
        if (straddle) {
          asm volatile("" ::: "memory");
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            if constexpr (packed)  // qs <= k_pos <= qpos as one unsigned compare
              sc[i] = ((uint32_t)kp[key] - (uint32_t)qs > (uint32_t)qpos - (uint32_t)qs)
                          ? -INFINITY : sc[i];
            else
              sc[i] = (kp[key] > qpos) ? -INFINITY : sc[i];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      // dP of block kb (V operands read LA ahead), the exponentials of its
      // scores between its contractions (P overwrites S in place)
      auto dprobs = [&](int kb, f32x16& sc) {
        const int rb = kb * 32 * D * 2;
        bf16x8 op[C::KS];
#pragma unroll
        for (int i = 0; i < LA; ++i) op[i] = lds_read_b128(vt, rb + koff[i]);
        f32x16 dp = dinit;
#pragma unroll
        for (int i = 0; i < C::KS; ++i) {
          if (i + LA < C::KS) op[i + LA] = lds_read_b128(vt, rb + koff[i + LA]);
          dp = mfma32x32x16(op[i], df[i], dp);
#pragma unroll
          for (int e = 0; e < EPM; ++e)
            sc[EPM * i + e] = fast_exp2(fmaf(sc[EPM * i + e], c, -lse2));
          __builtin_amdgcn_sched_barrier(0);
        }
        return dp;
      };
      // dQ^T += K^T dS^T for block kb
      auto dq_update = [&](int kb, const uint32_t (&dsk)[8]) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const u32x4 bw = {dsk[4 * half], dsk[4 * half + 1], dsk[4 * half + 2],
                            dsk[4 * half + 3]};
          const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
          const int rk = (2 * kb + half) * 16 * D * 2;
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb)
            dqacc[mb] = mfma32x32x16(lds_read_tr(kt, rk + troff[0][mb], rk + troff[1][mb]), b,
                                     dqacc[mb]);
        }
      };
      // block 0: S, mask, dP with the exponentials; block 1's S then runs
      // with block 0's dS between its contractions
      if (!packed) issue_tile(t + 1, Next{}, more);
      f32x16 s0 = scores(0, [](int) {});
      mask(0, s0);
      f32x16 dp0 = dprobs(0, s0);
      uint32_t dsk0[8];
      f32x16 s1 = scores(1, [&](int i) {
#pragma unroll
        for (int e = 0; e < EPM; e += 2)
          dsk0[(EPM * i + e) >> 1] = pack_bf16x2(s0[EPM * i + e] * dp0[EPM * i + e],
                                                 s0[EPM * i + e + 1] * dp0[EPM * i + e + 1]);
      });
      dq_update(0, dsk0);
      mask(1, s1);
      f32x16 dp1 = dprobs(1, s1);
      uint32_t dsk1[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) dsk1[i >> 1] = pack_bf16x2(s1[i] * dp1[i], s1[i + 1] * dp1[i + 1]);
      dq_update(1, dsk1);
    }
    if (more) {
      if (tid < C::BN) kpos_of(Next{})[tid] = key_live ? kpreg : kPosInf;
      wait_vmem();
    }
    __syncthreads();
  };

  if (nt > 0) {
    issue_tile(0, B0{}, true);
    if (tid < C::BN) sKp0[tid] = key_live ? kpreg : kPosInf;
    wait_vmem();
  }
  __syncthreads();
  for (int t = 0; t < nt; t += 2) {
    step(B0{}, t);
    if (t + 1 < nt) step(B1{}, t + 1);
  }

  // ---- epilogue: dq_acc += scale * (dQ^T)^T (this lane owns its elements) ----
  if (!row_ok || nt == 0) return;
  float* dqr = p.dq + ((size_t)row * p.hq + h) * D;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = mb * 32 + 8 * g + 4 * hh;
      f32x4 v = *(const f32x4*)(dqr + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(p.scale, dqacc[mb][4 * g + e], v[e]);
      *(f32x4*)(dqr + d0) = v;
    }
}


template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  // packed samples get their own instances so the plain causal path carries
  // no sample-start loads, compares or bounds
  const bool packed = p.q_start != nullptr;
  if (p.run_dkdv) {
    if (packed)
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, true>), dim3(p.n_ktiles * p.hkv), dim3(256), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, false>), dim3(p.n_ktiles * p.hkv), dim3(256),
                         0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!p.run_dq) return hipSuccess;
  if (packed)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, true>), dim3(p.n_qtiles * p.hq), dim3(256), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, false>), dim3(p.n_qtiles * p.hq), dim3(256), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace

static_assert(DkdvCfg<64>::BK == DkdvCfg<128>::BK && DkdvCfg<64>::BQ == DkdvCfg<128>::BQ &&
                  DqCfg<64>::BM == DqCfg<128>::BM && DqCfg<64>::BN == DqCfg<128>::BN,
              "tile plans are laid out for one tile shape per kernel");
int bwd_keys_per_block() { return DkdvCfg<128>::BK; }
int bwd_rows_per_block() { return DqCfg<128>::BM; }
int dkdv_rows_per_tile() { return DkdvCfg<128>::BQ; }
int dq_keys_per_tile() { return DqCfg<128>::BN; }

hipError_t launch_attn_bwd(const BwdParams& p, int d, hipStream_t stream) {
  return d == 64 ? launch_bwd_d<64>(p, stream) : launch_bwd_d<128>(p, stream);
}

}  // namespace mmsp
