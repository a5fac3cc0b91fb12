// Backward of causal attention of a query shard against one KV chunk (gfx950).
//
// The pages train at 2M tokens without gradient checkpointing ("LongVILA -
// ... (Jason's Study)", section "What it is"), so the backward consumes the
// forward's saved output and log-sum-exp: P = exp(scale q.k - LSE_final) on
// visible pairs, dV = P^T dO, dS = P o (dO V^T - delta), dQ += scale dS K,
// dK = scale dS^T Q, with dK/dV of a KV head summed over its query heads.
//
// Design (one workgroup = 128 keys of one KV head, 4 waves of 32 keys):
//  * K and V of the wave's 32 keys stay in registers (B operands of
//    S = Q K^T and dP = dO V^T); the dK^T and dV^T accumulators too;
//  * the workgroup walks the visible query tiles (32 rows) of every query
//    head of its KV head; each tile's Q and dO are prefetched into registers
//    one tile ahead and stored to double-buffered LDS both row-major (A of S
//    and dP) and transposed in kPerm16 order (A of dK^T and dV^T, whose B
//    operands are the P / dS accumulators reused in place);
//  * dS (bf16) goes through LDS once so the four waves can form
//    dQ = dS K over all 128 keys (each wave one 32-wide slice of the head
//    dim) and add it to dq with fp32 atomics (two 128-byte lines per
//    instruction);
//  * causal skipping: the query range of a workgroup starts at the first
//    query that can see its first key (binary search); a wave skips tiles it
//    cannot see and masks only straddling tiles.
#include "common.h"
#include "kernels.h"

namespace mmsp {
namespace {

template <int D>
struct BwdCfg {
  static constexpr int BK = 128;          // keys per workgroup
  static constexpr int BQ = 32;           // queries per tile
  static constexpr int THREADS = 256;
  static constexpr int KS = D / 16;       // K-steps over the head dim
  static constexpr int MB = D / 32;       // 32-row blocks of the head dim
  static constexpr int CPR = D / 8;       // 16-byte chunks per row
  static constexpr int RSTR = D + 8;      // [q][d] stride (bf16)
  static constexpr int TSTR = BQ + 8;     // [d][q] stride (bf16)
  static constexpr int KTSTR = BK + 8;    // K^T [d][key] stride (bf16)
  static constexpr int SSTR = BK + 8;     // dS [q][key] stride (bf16)
  static constexpr int QITEMS = (BQ / 4) * CPR;  // (4 rows x 8 dims) items per tensor
};

constexpr int kPosInf = 0x7fffffff;

// 4 rows x 8 bf16 (one u32x4 per row) -> 8 rows of 4 bf16, written at
// base[e * stride] for e = 0..7 (the transposed layout's 8 head-dim rows).
__device__ __forceinline__ void store_transposed_4x8(uint16_t* base, int stride, const u32x4* r) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    const uint32_t a0 = r[0][w], a1 = r[1][w], a2 = r[2][w], a3 = r[3][w];
    u32x2 out;
    if ((e & 1) == 0) {
      out[0] = (a0 & 0xffffu) | (a1 << 16);
      out[1] = (a2 & 0xffffu) | (a3 << 16);
    } else {
      out[0] = (a0 >> 16) | (a1 & 0xffff0000u);
      out[1] = (a2 >> 16) | (a3 & 0xffff0000u);
    }
    *(u32x2*)(base + e * stride) = out;
  }
}

template <int D>
__global__ void __launch_bounds__(256, 1) attn_bwd_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t sKt[D * C::KTSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][C::BQ * C::RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[2][C::BQ * C::RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sQt[2][D * C::TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sdOt[2][D * C::TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sdS[2][C::BQ * C::SSTR];
  __shared__ __attribute__((aligned(16))) float sL[2][C::BQ];   // LSE * log2e (+inf if empty)
  __shared__ __attribute__((aligned(16))) float sDl[2][C::BQ];  // delta
  __shared__ __attribute__((aligned(16))) int sQp[2][C::BQ];    // positions (INT_MIN past sq)
  __shared__ int sQlast[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int kvh = logical / p.n_ktiles;
  const int kt = logical % p.n_ktiles;  // early keys (more visible queries) first
  const int j0 = kt * C::BK;
  const int key = j0 + wave * 32 + l32;  // this lane's key
  const bool key_ok = key < p.sk;
  const size_t kv_stride = (size_t)p.hkv * D;

  // ---- key positions of the lane / wave / workgroup ----
  const int kpos = key_ok ? (p.causal ? p.k_pos[key] : 0) : kPosInf;
  const int wk0 = j0 + wave * 32;
  const bool wave_live = wk0 < p.sk;
  const int wk_last = min(wk0 + 31, p.sk - 1);
  const bool wave_full_keys = wk0 + 31 < p.sk;
  int wkmin = kPosInf, wkmax = kPosInf;
  if (wave_live) {
    wkmin = p.causal ? p.k_pos[wk0] : 0;
    wkmax = p.causal ? p.k_pos[wk_last] : 0;
  }
  // first query that can see the workgroup's first key
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
  const int n_qt = (p.sq + C::BQ - 1) / C::BQ;
  const int qt0 = qstart / C::BQ;
  const int per_head = n_qt - qt0;
  const int total = per_head > 0 ? per_head * p.group : 0;

  // ---- stationary K, V fragments (B operands, col = key, k = head dim) ----
  bf16x8 kf[C::KS], vf[C::KS];
  {
    const uint16_t* kr = p.k + (size_t)key * kv_stride + (size_t)kvh * D + 8 * hh;
    const uint16_t* vr = p.v + (size_t)key * kv_stride + (size_t)kvh * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key_ok) {
        a = *(const u32x4*)(kr + 16 * ks);
        b = *(const u32x4*)(vr + 16 * ks);
      }
      kf[ks] = __builtin_bit_cast(bf16x8, a);
      vf[ks] = __builtin_bit_cast(bf16x8, b);
    }
  }
  // K^T of the workgroup's keys in LDS (natural key order) for dQ = dS K
  for (int it = tid; it < (C::BK / 4) * C::CPR; it += C::THREADS) {
    const int kg = it / C::CPR, dc = it % C::CPR;
    u32x4 r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j0 + 4 * kg + e;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (j < p.sk) w = *(const u32x4*)(p.k + (size_t)j * kv_stride + (size_t)kvh * D + dc * 8);
      r[e] = w;
    }
    store_transposed_4x8(&sKt[(8 * dc) * C::KTSTR + 4 * kg], C::KTSTR, r);
  }

  // ---- query-tile staging ----
  // threads [0, QITEMS) carry Q, [128, 128 + QITEMS) carry dO: 4 rows x 16 B
  u32x4 treg[4];
  float lreg = 0.f, dreg = 0.f;
  int preg = INT_MIN;
  const bool is_q = tid < 128;
  const int item = is_q ? tid : tid - 128;
  const bool item_ok = item < C::QITEMS;
  const int rg = item / C::CPR, dc = item % C::CPR;

  auto tile_of = [&](int it, int& h, int& q0) {
    const int gi = it / per_head;
    h = kvh * p.group + gi;
    q0 = (qt0 + it % per_head) * C::BQ;
  };
  auto load_tile = [&](int it) {
    int h, q0;
    tile_of(it, h, q0);
    if (item_ok) {
      const uint16_t* src = is_q ? p.q : p.dout;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = q0 + 4 * rg + e;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (i < p.sq) w = *(const u32x4*)(src + ((size_t)i * p.hq + h) * D + dc * 8);
        treg[e] = w;
      }
    }
    if (tid < C::BQ) {
      const int i = q0 + tid;
      if (i < p.sq) {
        const float l = p.lse[(size_t)h * p.sq + i];
        lreg = (l == -INFINITY) ? INFINITY : l * kLog2e;
        dreg = p.delta[(size_t)h * p.sq + i];
        preg = p.causal ? p.q_pos[i] : (kPosInf - 1);
      } else {
        lreg = INFINITY;
        dreg = 0.f;
        preg = INT_MIN;
      }
    }
    if (tid == C::BQ) {
      const int last = min(q0 + C::BQ - 1, p.sq - 1);
      preg = p.causal ? p.q_pos[last] : (kPosInf - 1);
    }
  };
  auto store_tile = [&](int buf) {
    if (item_ok) {
      uint16_t* rm = is_q ? sQ[buf] : sdO[buf];
      uint16_t* tr = is_q ? sQt[buf] : sdOt[buf];
#pragma unroll
      for (int e = 0; e < 4; ++e) *(u32x4*)&rm[(4 * rg + e) * C::RSTR + dc * 8] = treg[e];
      const int q = 4 * rg;
      const int col = (q & ~15) + kPerm16(q & 15);
      store_transposed_4x8(&tr[(8 * dc) * C::TSTR + col], C::TSTR, treg);
    }
    if (tid < C::BQ) {
      sL[buf][tid] = lreg;
      sDl[buf][tid] = dreg;
      sQp[buf][tid] = preg;
    }
    if (tid == C::BQ) sQlast[buf] = preg;
  };

  f32x16 dkacc[C::MB], dvacc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    dkacc[mb] = f32x16{};
    dvacc[mb] = f32x16{};
  }
  const float c = p.scale_log2;

  if (total > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int buf = it & 1;
    if (it + 1 < total) load_tile(it + 1);
    int h, q0;
    tile_of(it, h, q0);
    const int qfirst = sQp[buf][0];
    const int qlast = sQlast[buf];
    uint16_t* ds_out = &sdS[buf][0];
    const bool vis = wave_live && qlast >= wkmin;
    if (vis) {
      const bool full = wave_full_keys && qfirst >= wkmax && (q0 + C::BQ <= p.sq);
      // S = Q K^T and dP = dO V^T  (row = query, col = key)
      f32x16 s = f32x16{}, dp = f32x16{};
      const uint16_t* qr = &sQ[buf][l32 * C::RSTR + 8 * hh];
      const uint16_t* dr = &sdO[buf][l32 * C::RSTR + 8 * hh];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(qr + 16 * ks));
        s = mfma32x32x16(a, kf[ks], s);
      }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(dr + 16 * ks));
        dp = mfma32x32x16(a, vf[ks], dp);
      }
      uint32_t pk[8], dsk[8];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int q = 8 * g + 4 * hh;  // rows q .. q+3 of this lane
        const f32x4 lq = *(const f32x4*)&sL[buf][q];
        const f32x4 dq = *(const f32x4*)&sDl[buf][q];
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pe = fast_exp2(fmaf(s[4 * g + e], c, -lq[e]));
          if (!full && kpos > sQp[buf][q + e]) pe = 0.f;
          pv[e] = pe;
          dsv[e] = pe * (dp[4 * g + e] - dq[e]);
        }
        pk[2 * g] = pack_bf16x2(pv[0], pv[1]);
        pk[2 * g + 1] = pack_bf16x2(pv[2], pv[3]);
        dsk[2 * g] = pack_bf16x2(dsv[0], dsv[1]);
        dsk[2 * g + 1] = pack_bf16x2(dsv[2], dsv[3]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS  (row = head dim, col = key, k = query)
#pragma unroll
      for (int ks = 0; ks < C::BQ / 16; ++ks) {
        const u32x4 pw = {pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
        const u32x4 sw = {dsk[4 * ks], dsk[4 * ks + 1], dsk[4 * ks + 2], dsk[4 * ks + 3]};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        const bf16x8 sb = __builtin_bit_cast(bf16x8, sw);
        const uint16_t* dot = &sdOt[buf][l32 * C::TSTR + 16 * ks + 8 * hh];
        const uint16_t* qt = &sQt[buf][l32 * C::TSTR + 16 * ks + 8 * hh];
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
          const bf16x8 a1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(dot + mb * 32 * C::TSTR));
          dvacc[mb] = mfma32x32x16(a1, pb, dvacc[mb]);
          const bf16x8 a2 = __builtin_bit_cast(bf16x8, *(const u32x4*)(qt + mb * 32 * C::TSTR));
          dkacc[mb] = mfma32x32x16(a2, sb, dkacc[mb]);
        }
      }
      // dS -> LDS as [query][key] (natural orders) for dQ = dS K
      const int kcol = wave * 32 + l32;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = dsk[2 * g + (e >> 1)];
          ds_out[(8 * g + 4 * hh + e) * C::SSTR + kcol] = (e & 1) ? (uint16_t)(w >> 16)
                                                                  : (uint16_t)(w & 0xffffu);
        }
    } else {
      const int kcol = wave * 32 + l32;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) ds_out[(8 * g + 4 * hh + e) * C::SSTR + kcol] = 0;
    }
    if (it + 1 < total) store_tile(buf ^ 1);
    __syncthreads();
    // dQ[q0 .. q0+32)[32*wave .. +32) += scale * dS K   (row = query, col = head dim);
    // every tile walked holds a query that sees the workgroup's first key
    if (wave < C::MB) {
      f32x16 acc = f32x16{};
      const uint16_t* ar = &sdS[buf][l32 * C::SSTR + 8 * hh];
      const uint16_t* br = &sKt[(wave * 32 + l32) * C::KTSTR + 8 * hh];
#pragma unroll
      for (int ks = 0; ks < C::BK / 16; ++ks) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(ar + 16 * ks));
        const bf16x8 b = __builtin_bit_cast(bf16x8, *(const u32x4*)(br + 16 * ks));
        acc = mfma32x32x16(a, b, acc);
      }
      float* dqb = p.dq + (size_t)h * D + wave * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = q0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (q < p.sq) atomicAdd(dqb + (size_t)q * p.hq * D, acc[i] * p.scale);
      }
    }
  }

  // ---- epilogue: dK = scale * dK^T^T, dV = dV^T^T ----
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

}  // namespace

int bwd_keys_per_block() { return BwdCfg<128>::BK; }

hipError_t launch_attn_bwd(const BwdParams& p, int d, hipStream_t stream) {
  const int grid = p.n_ktiles * p.hkv;
  if (d == 64)
    hipLaunchKernelGGL(attn_bwd_kernel<64>, dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_bwd_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mmsp
