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
// bounded by a binary search on the sorted positions, waves skip tiles they
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
  __shared__ __attribute__((aligned(16))) float sL[2][C::BQ];      // LSE*log2e (+inf empty)
  __shared__ __attribute__((aligned(16))) float sDl[2][C::BQ];     // delta
  __shared__ __attribute__((aligned(16))) int sQp[2][C::BQ];       // positions
  __shared__ __attribute__((aligned(16))) int sQs[2][C::BQ];       // sample starts (packed)
  __shared__ int sQlast[2];
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
  const int kvh = logical / p.n_ktiles;
  // early keys see more queries: their end of the range is dispatched first
  const int kt = p.n_ktiles - 1 - heavy_first_tile(logical % p.n_ktiles, p.n_ktiles, gridDim.x);
  const int j0 = kt * C::BK;
  const int key = j0 + wave * 32 + l32;
  const bool key_ok = key < p.sk;
  const size_t kv_stride = (size_t)p.hkv * D;

  const int kpos = key_ok ? (p.causal ? p.k_pos[key] : 0) : kPosInf;
  const int wk0 = j0 + wave * 32;
  const bool wave_live = wk0 < p.sk;
  const bool wave_full_keys = wk0 + 31 < p.sk;
  int wkmin = kPosInf, wkmax = kPosInf;
  if (wave_live) {
    wkmin = p.causal ? p.k_pos[wk0] : 0;
    wkmax = p.causal ? p.k_pos[min(wk0 + 31, p.sk - 1)] : 0;
  }
  wkmin = uniform(wkmin);
  wkmax = uniform(wkmax);
  int qstart = 0;
  if (p.causal) {
    const int kmin = p.k_pos[j0];
    int lo = 0, hi = p.sq;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (p.q_pos[mid] < kmin) lo = mid + 1; else hi = mid;
    }
    qstart = lo;
  }
  // packed samples: only queries whose sample starts at or before the
  // workgroup's last key can see it (sample starts are non-decreasing)
  constexpr bool packed = PACKED;  // q_start given
  int qend = p.sq;
  if (packed) {
    const int kmax = p.k_pos[min(j0 + C::BK - 1, p.sk - 1)];
    int lo = 0, hi = p.sq;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (p.q_start[mid] <= kmax) lo = mid + 1; else hi = mid;
    }
    qend = lo;
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
  const uint32_t* stat_src = wave == 0   ? (const uint32_t*)p.q_start
                             : wave == 1 ? (const uint32_t*)p.lse
                             : wave == 2 ? (const uint32_t*)p.delta
                             : p.causal  ? (const uint32_t*)p.q_pos
                                         : (const uint32_t*)p.lse;  // any readable row
  const size_t stat_head = (wave == 1 || wave == 2) ? (size_t)p.sq : 0;
  auto issue_next = [&](auto buf) {
    const int h = nx_h, q0 = nx_q0;
    const size_t o = nx_off;
    nx_q0 += C::BQ;
    nx_off += tile_step;
    if (nx_q0 >= n_qt * C::BQ) {
      nx_q0 = qt0 * C::BQ;
      ++nx_h;
      nx_off -= head_back;
    }
    if (q0 + C::BQ <= p.sq) {
      ld.load(qtile(buf), p.q + o);
      ld.load(otile(buf), p.dout + o);
    } else {
      ld.load_clamped(qtile(buf), p.q + o, q_row_stride, p.sq - q0);
      ld.load_clamped(otile(buf), p.dout + o, q_row_stride, p.sq - q0);
    }
    // Raw values only: they are converted when published, after the wait
    // that ends the step, so no load here is waited for inside the step.
    if ((wave != 0 || packed) && lane <= C::BQ) {
      const int i = min(q0 + min(lane, C::BQ - 1), p.sq - 1);
      stat = stat_src[(size_t)h * stat_head + i];
      row_live = q0 + lane < p.sq;
    }
  };
  auto publish_tile = [&](int buf) {
    if (wave == 0 && lane < C::BQ) {
      sQs[buf][lane] = (packed && row_live) ? (int)stat : INT_MIN;
    } else if (wave == 1 && lane < C::BQ) {
      // empty rows (LSE = -inf) and rows past sq get P = exp2(s c - inf) = 0
      const float l = __uint_as_float(stat);
      sL[buf][lane] = (row_live && l != -INFINITY) ? l * kLog2e : INFINITY;
    } else if (wave == 2 && lane < C::BQ) {
      sDl[buf][lane] = row_live ? __uint_as_float(stat) : 0.f;
    } else if (wave == 3 && lane <= C::BQ) {
      const int pos = p.causal ? (int)stat : kPosInf - 1;
      if (lane < C::BQ) sQp[buf][lane] = row_live ? pos : INT_MIN;
      else sQlast[buf] = pos;
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
    if (it + 1 < total) issue_next(Next{});
    const lds_char* qt = qtile(buf_tag);
    const lds_char* dt = otile(buf_tag);
    const int qfirst = uniform(sQp[BUF][0]);
    const int qlast = uniform(sQlast[BUF]);
    const int qs_first = packed ? uniform(sQs[BUF][0]) : INT_MIN;
    const int qs_last = packed ? uniform(sQs[BUF][C::BQ - 1]) : INT_MIN;
    if (wave_live && qlast >= wkmin && qs_first <= wkmax) {
      // S = Q K^T and dP = dO V^T  (row = query, col = key)
      f32x16 s = mfma32x32x16(lds_read_b128(qt, qoff[0]), kf[0], f32x16{});
      f32x16 dp = mfma32x32x16(lds_read_b128(dt, qoff[0]), lds_read_b128(vrows, qoff[0]),
                               f32x16{});
#pragma unroll
      for (int ks = 1; ks < C::KS; ++ks) {
        s = mfma32x32x16(lds_read_b128(qt, qoff[ks]), kf[ks], s);
        dp = mfma32x32x16(lds_read_b128(dt, qoff[ks]), lds_read_b128(vrows, qoff[ks]), dp);
      }
      const int last_row_pos = uniform(sQp[BUF][C::BQ - 1]);  // INT_MIN past sq
      // straddles the rows' positions or their sample starts (or the tail)
      if (!(wave_full_keys && qfirst >= wkmax && last_row_pos != INT_MIN && qs_last <= wkmin)) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = 8 * (i >> 2) + 4 * hh + (i & 3);
          bool hide = kpos > sQp[BUF][q];
          if constexpr (packed) hide |= kpos < sQs[BUF][q];
          s[i] = hide ? -INFINITY : s[i];
        }
      }
      uint32_t pk[8], dsk[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int q = 8 * g + 4 * hh;  // rows q .. q+3 of this lane
        const f32x4 lq = *(const f32x4*)&sL[BUF][q];
        const f32x4 dq = *(const f32x4*)&sDl[BUF][q];
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = fast_exp2(fmaf(s[4 * g + e], c, -lq[e]));
          pv[e] = pe;
          dsv[e] = pe * (dp[4 * g + e] - dq[e]);
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
    if (it + 1 < total) {
      publish_tile(BUF ^ 1);
      wait_vmem();
    }
    __syncthreads();
  };

  if (total > 0) {
    issue_next(B0{});
    publish_tile(0);
  }
  wait_vmem();
  __syncthreads();
  for (int it = 0; it < total; it += 2) {
    step(B0{}, it);
    if (it + 1 < total) step(B1{}, it + 1);
  }

  // ---- epilogue: dK = scale * (dK^T)^T, dV = (dV^T)^T ----
  if (!key_ok) return;
  float* dkr = p.dk + (size_t)key * kv_stride + (size_t)kvh * D;
  float* dvr = p.dv + (size_t)key * kv_stride + (size_t)kvh * D;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = mb * 32 + 8 * g + 4 * hh;
      f32x4 kv4 = {dkacc[mb][4 * g] * p.scale, dkacc[mb][4 * g + 1] * p.scale,
                   dkacc[mb][4 * g + 2] * p.scale, dkacc[mb][4 * g + 3] * p.scale};
      f32x4 vv4 = {dvacc[mb][4 * g], dvacc[mb][4 * g + 1], dvacc[mb][4 * g + 2],
                   dvacc[mb][4 * g + 3]};
      if (p.accumulate) {
        kv4 += *(const f32x4*)(dkr + d0);
        vv4 += *(const f32x4*)(dvr + d0);
      }
      *(f32x4*)(dkr + d0) = kv4;
      *(f32x4*)(dvr + d0) = vv4;
    }
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
  const int h = logical / p.n_qtiles;
  const int qt = heavy_first_tile(logical % p.n_qtiles, p.n_qtiles, gridDim.x);
  const int kvh = h / p.group;
  const int q0 = qt * C::BM;
  const int row = q0 + wave * 32 + l32;
  const bool row_ok = row < p.sq;

  int qpos = INT_MIN;
  float lse2 = INFINITY, delta = 0.f;
  if (row_ok) {
    qpos = p.causal ? p.q_pos[row] : (kPosInf - 1);
    const float l = p.lse[(size_t)h * p.sq + row];
    lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    delta = p.delta[(size_t)h * p.sq + row];
  }
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
  // packed samples: keys below a row's sample start are hidden too
  constexpr bool packed = PACKED;  // q_start given
  const int qs = (packed && row_ok) ? p.q_start[row] : INT_MIN;
  const int wqs_min = uniform((packed && wave_live) ? p.q_start[wr0] : INT_MIN);
  const int wqs_max =
      uniform((packed && wave_live) ? p.q_start[min(wr0 + 31, p.sq - 1)] : INT_MIN);
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
  auto issue_tile = [&](int t, auto buf) {
    const int j0 = (tb + t) * C::BN;
    const size_t o = (size_t)j0 * kv_row_stride;
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
  };

  f32x16 dqacc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) dqacc[mb] = f32x16{};
  const float c = p.scale_log2;

  auto step = [&](auto buf_tag, int t) {
    constexpr int BUF = decltype(buf_tag)::value;
    using Next = std::integral_constant<int, BUF ^ 1>;
    if (t + 1 < nt) issue_tile(t + 1, Next{});
    const lds_char* kt = ktile(buf_tag);
    const lds_char* vt = vtile(buf_tag);
    const int* kp = kpos_of(buf_tag);
    const int kfirst = uniform(kp[0]);
    const int klast = uniform(kp[C::BN - 1]);
    if (wave_live && kfirst <= wqmax && klast >= wqs_min) {
      // straddles the rows' positions or their sample starts
      const bool straddle = klast > wqmin || kfirst < wqs_max;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {  // 32 keys at a time
        const int rb = kb * 32 * D * 2;
        f32x16 s = mfma32x32x16(lds_read_b128(kt, rb + koff[0]), qf[0], f32x16{});
        f32x16 dp = mfma32x32x16(lds_read_b128(vt, rb + koff[0]), df[0], f32x16{});
#pragma unroll
        for (int ks = 1; ks < C::KS; ++ks) {
          s = mfma32x32x16(lds_read_b128(kt, rb + koff[ks]), qf[ks], s);
          dp = mfma32x32x16(lds_read_b128(vt, rb + koff[ks]), df[ks], dp);
        }
        if (straddle) {
          asm volatile("" ::: "memory");
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
            if constexpr (packed)  // qs <= k_pos <= qpos as one unsigned compare
              s[i] = ((uint32_t)kp[key] - (uint32_t)qs > (uint32_t)qpos - (uint32_t)qs)
                         ? -INFINITY : s[i];
            else
              s[i] = (kp[key] > qpos) ? -INFINITY : s[i];
          }
        }
        uint32_t dsk[8];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = fast_exp2(fmaf(s[i], c, -lse2));
          const float p1 = fast_exp2(fmaf(s[i + 1], c, -lse2));
          dsk[i >> 1] = pack_bf16x2(p0 * (dp[i] - delta), p1 * (dp[i + 1] - delta));
        }
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
      }
    }
    if (t + 1 < nt) {
      if (tid < C::BN) kpos_of(Next{})[tid] = key_live ? kpreg : kPosInf;
      wait_vmem();
    }
    __syncthreads();
  };

  if (nt > 0) {
    issue_tile(0, B0{});
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

int bwd_keys_per_block() { return DkdvCfg<128>::BK; }
int bwd_rows_per_block() { return DqCfg<128>::BM; }

hipError_t launch_attn_bwd(const BwdParams& p, int d, hipStream_t stream) {
  return d == 64 ? launch_bwd_d<64>(p, stream) : launch_bwd_d<128>(p, stream);
}

}  // namespace mmsp
