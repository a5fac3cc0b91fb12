// Device helpers shared by the gfx950 kernels of libmmsp.so.
//
// Matrix-core conventions (CDNA4 v_mfma_f32_32x32x16_bf16, 64-lane wave):
//   A (32 x 16, M x K): lane l supplies row m = l % 32, k = 8*(l/32) + 0..7
//   B (16 x 32, K x N): lane l supplies col n = l % 32, k = 8*(l/32) + 0..7
//   C (32 x 32, fp32) : lane l holds col n = l % 32 and, for i = 0..15,
//                       row m = 8*(i/4) + 4*(l/32) + (i%4)
// A C tile fed back as the B operand of the next contraction (its row index
// becoming K) supplies, in K-step 0, rows {0-3, 8-11} from lane-half 0 and
// rows {4-7, 12-15} from lane-half 1 (entries 0..7), and the same +16 in
// K-step 1 (entries 8..15).  The paired A operand must list its K rows in
// that order; the transposing LDS read below produces exactly that order.
//
// LDS tiles: rows of D bf16 (row-major, no padding) whose 16-byte chunks are
// XOR-swizzled, chunk c of row r stored at chunk slot c ^ swz(r).  With
// swz(r) = ((r & 3) << 2) | ((r >> 2) & 3) (D = 128) both access patterns used
// here are free of bank conflicts: 16 lanes reading one chunk of 16
// consecutive rows (ds_read_b128), and the transposing read of 4 rows x 4
// chunks per 32 lanes (ds_read_b64_tr_b16).  Tiles are filled by direct
// buffer->LDS loads (buffer_load_dwordx4 ... lds): lane l of a wave writes LDS
// bytes [16 l, 16 l + 16) of the wave's 1 KiB window, so the swizzle is
// applied by choosing which global chunk each lane fetches.  The buffer
// (MUBUF) form is used rather than global_load_lds: a FLAT-encoded load in
// flight makes the compiler treat LDS reads as completing out of order, so it
// would wait for all of them (lgkmcnt(0)) before every use instead of only
// for the one being consumed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmsp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPosInf = 0x7fffffff;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// acc + lo(w) + hi(w) for a packed bf16 pair (v_dot2c_f32_bf16 against 1.0)
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// max / sum of a value with the same lane in the other half of the wave
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Workgroup order that keeps consecutive logical tiles on one XCD: the
// dispatcher deals workgroup b to XCD b % 8, so logical tile
// (b % 8) * (n / 8) + b / 8 runs on XCD b % 8 and each XCD sweeps one
// contiguous range of logical tiles (sharing its L2).
__device__ __forceinline__ int xcd_logical_block(int b, int n) {
  if ((n & 7) != 0) return b;
  return (b & 7) * (n >> 3) + (b >> 3);
}

// Order of the n tiles of one head, given the dispatch index i within the
// head, so that the heavy end (tile n-1: late queries, or early keys once the
// caller reverses it) is dispatched first.
//
// When one head's tiles fill less than an XCD's share of the grid (each XCD
// runs a contiguous range of logical tiles), whole heads share an XCD and the
// plain heavy-first order is used.  When a head spans several XCDs, a plain
// order would hand one XCD only heavy tiles and the next only light ones (the
// two blocks of a zigzag shard: one may see none of a chunk), so the order
// alternates between the two ends in blocks of 8 tiles: blocks n/8-1, 0,
// n/8-2, 1, ... each in natural order.  Runs of 8 keep consecutive
// workgroups -- which the dispatcher deals to different shader engines of an
// XCD -- of one kind, so no engine collects only the heavy tiles.
__device__ __forceinline__ int heavy_first_tile(int i, int n, int grid) {
  if ((n << 3) <= grid || (n & 7) != 0) return n - 1 - i;
  const int nb = n >> 3, bi = i >> 3;
  const int blk = (bi & 1) ? (bi >> 1) : nb - 1 - (bi >> 1);
  return (blk << 3) | (i & 7);
}

// Lengths of the prefixes of two non-decreasing arrays on which a predicate
// holds: a[i] < xa (or <= xa with LE_A) and b[i] < xb (or <= xb with LE_B).
// Each round every lane of the wave probes one entry of each unresolved range
// and a ballot finds where the predicate turns false, so a range shrinks
// 64-fold per round: 8192 entries take three rounds (one load each, the two
// searches side by side) instead of thirteen dependent loads.  Call with the
// whole wave active; results are wave-uniform.
template <bool LE_A, bool LE_B>
__device__ __forceinline__ void wave_prefix_two(const int32_t* a, int na, int xa, const int32_t* b,
                                                int nb, int xb, int& ca, int& cb) {
  const int lane = (int)(threadIdx.x & 63);
  int alo = 0, ahi = na, blo = 0, bhi = nb;
  while (alo < ahi || blo < bhi) {
    const int as = (ahi - alo + 63) >> 6, bs = (bhi - blo + 63) >> 6;
    const int ai = alo + (lane + 1) * as - 1, bi = blo + (lane + 1) * bs - 1;
    bool aok = false, bok = false;
    if (as > 0 && ai < ahi) {  // a resolved range (as == 0) is not probed
      const int v = a[ai];
      aok = LE_A ? v <= xa : v < xa;
    }
    if (bs > 0 && bi < bhi) {
      const int v = b[bi];
      bok = LE_B ? v <= xb : v < xb;
    }
    // the predicate holds on a prefix of the probes: lanes [0, n)
    const int an = __popcll(__ballot(aok)), bn = __popcll(__ballot(bok));
    const int af = alo + (an + 1) * as - 1, bf = blo + (bn + 1) * bs - 1;  // first failing probe
    ahi = uniform((as > 0 && an < 64 && af < ahi) ? af : ahi);
    bhi = uniform((bs > 0 && bn < 64 && bf < bhi) ? bf : bhi);
    alo = uniform(min(alo + an * as, ahi));
    blo = uniform(min(blo + bn * bs, bhi));
  }
  ca = alo;
  cb = blo;
}

// wave_prefix_two for one array.
template <bool LE>
__device__ __forceinline__ int wave_prefix(const int32_t* a, int n, int x) {
  const int lane = (int)(threadIdx.x & 63);
  int lo = 0, hi = n;
  while (lo < hi) {
    const int st = (hi - lo + 63) >> 6;
    const int i = lo + (lane + 1) * st - 1;
    bool ok = false;
    if (i < hi) {
      const int v = a[i];
      ok = LE ? v <= x : v < x;
    }
    const int k = __popcll(__ballot(ok));
    const int f = lo + (k + 1) * st - 1;
    hi = uniform((k < 64 && f < hi) ? f : hi);
    lo = uniform(min(lo + k * st, hi));
  }
  return lo;
}

// Head and tile of workgroup b from a work-ordered tile list (heaviest first)
// of n tiles per head, H heads.  As with xcd_logical_block, each XCD keeps a
// contiguous share of the heads (with H a multiple of 8); within it the heads
// take turns, so every XCD starts with the heaviest tiles of all its heads
// and ends with the lightest.  Otherwise heads simply take turns.  A list
// entry outside [0, n) is clamped (a damaged list can give wrong results,
// never an access out of bounds).
__device__ __forceinline__ void planned_tile(int b, int n, int H, const int32_t* list, int& h,
                                             int& t) {
  int j;
  if ((H & 7) == 0) {
    const int hx = H >> 3;
    j = (b >> 3) / hx;
    h = (b & 7) * hx + (b >> 3) % hx;
  } else {
    j = b / H;
    h = b % H;
  }
  t = min(max(uniform(list[j]), 0), n - 1);
}

// Whether a tile plan (layout in kernels.h) was made for these sizes.
__device__ __forceinline__ bool plan_fits(const int32_t* plan, int32_t magic, int sq, int sk) {
  if (plan == nullptr) return false;
  return uniform(plan[0]) == magic && uniform(plan[1]) == sq && uniform(plan[2]) == sk;
}

// ---- swizzled LDS tiles -----------------------------------------------------
template <int D>
__device__ __forceinline__ constexpr int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// byte offset of (row, 16-byte chunk c) in a swizzled tile of rows of D bf16
template <int D>
__device__ __forceinline__ int tile_off(int row, int c) {
  return row * (D * 2) + ((c ^ swz<D>(row)) << 4);
}

// Buffer resource over [base, base + nbytes) (raw, stride 0; gfx9 dword 3 =
// 32-bit data format).  Base and size are taken from lane 0: callers pass
// wave-uniform values, and reading them through readfirstlane keeps the
// descriptor in scalar registers without a waterfall loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = (uint64_t)base;
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const int n = __builtin_amdgcn_readfirstlane((int)nbytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)u, (short)0, n, 0x00020000);
}

__device__ __forceinline__ uint32_t clamp_bytes(size_t n) {
  return n > 0xffffffffull ? 0xffffffffu : (uint32_t)n;
}

// Direct LDS fill from a buffer: lane l writes SIZE bytes at dst + SIZE * l
// (dst wave-uniform), read from byte voff of the buffer; lanes whose voff is
// out of the buffer's range write zeros.
template <int SIZE>
__device__ __forceinline__ void buffer_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                              lds_char* dst) {
  static_assert(SIZE == 16 || SIZE == 4, "direct LDS load of 4 or 16 bytes per lane");
  auto* d = (__attribute__((address_space(3))) void*)dst;
  if constexpr (SIZE == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff, 0, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 4, voff, 0, 0, 0);
}

// Direct buffer->LDS fill of a ROWS x D bf16 tile by THREADS threads.
// Tile row r lives at global element offset r * row_stride from `base`.
// Per-lane byte offsets (loop invariant) index a buffer descriptor built on
// the wave-uniform tile base.
template <int D, int ROWS, int THREADS>
struct TileLoader {
  static constexpr int CPR = D / 8;
  static constexpr int ROUNDS = ROWS * CPR / THREADS;
  static_assert((ROWS * CPR) % THREADS == 0, "tile must be a whole number of load rounds");
  uint32_t off[ROUNDS];   // byte offset of this lane's chunk, row 0 = tile row 0
  int row[ROUNDS];        // tile row of this lane's chunk in each round
  int wave_base;
  size_t row_bytes;       // global bytes between consecutive tile rows

  __device__ __forceinline__ void init(int tid, size_t row_stride) {
    wave_base = uniform((tid >> 6) << 6);
    row_bytes = row_stride * 2;
    const int lane = tid & 63;
#pragma unroll
    for (int c = 0; c < ROUNDS; ++c) {
      const int slot = c * THREADS + wave_base + lane;
      const int r = slot / CPR;
      const int chunk = (slot % CPR) ^ swz<D>(r);
      row[c] = r;
      off[c] = (uint32_t)(((size_t)r * row_stride + chunk * 8) * 2);
    }
  }
  // all rows of the tile exist: base points at tile row 0
  __device__ __forceinline__ void load(lds_char* tile, const uint16_t* base) const {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, clamp_bytes((size_t)ROWS * row_bytes));
#pragma unroll
    for (int c = 0; c < ROUNDS; ++c) buffer_to_lds<16>(rs, off[c], tile + (c * THREADS + wave_base) * 16);
  }
  // the first `rows` rows of the tile; the rows after them lie outside the
  // buffer's range and arrive as zeros
  __device__ __forceinline__ void load_rows(lds_char* tile, const uint16_t* base, int rows) const {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, clamp_bytes((size_t)rows * row_bytes));
#pragma unroll
    for (int c = 0; c < ROUNDS; ++c) buffer_to_lds<16>(rs, off[c], tile + (c * THREADS + wave_base) * 16);
  }
  // tail tile: rows at or past `rows_left` re-read the last existing row
  __device__ __forceinline__ void load_clamped(lds_char* tile, const uint16_t* base,
                                               size_t row_stride, int rows_left) const {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, clamp_bytes((size_t)rows_left * row_bytes));
#pragma unroll
    for (int c = 0; c < ROUNDS; ++c) {
      const int back = row[c] - min(row[c], rows_left - 1);
      buffer_to_lds<16>(rs, off[c] - (uint32_t)((size_t)back * row_stride * 2),
                        tile + (c * THREADS + wave_base) * 16);
    }
  }
};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier without the memory fence of __syncthreads(): callers make
// their own LDS traffic visible first (wait_vmem_le for direct loads,
// lgkmcnt for ds writes), so in-flight prefetches of later tiles stay in flight.
__device__ __forceinline__ void barrier_only() { __builtin_amdgcn_s_barrier(); }

__device__ __forceinline__ void wait_lds_writes() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The same wait through the builtin: the compiler's own wait insertion sees
// it and does not wait again for the loads it retired.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 64 key positions of a tile straight into this wave's LDS slot (lane l ->
// slot[l]); rows at or past `valid` re-read the last existing position (the
// caller masks them by index).
__device__ __forceinline__ void pos_load_direct(lds_char* slot, const int32_t* src, int j0,
                                                int valid) {
  const int l = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src + j0, (uint32_t)valid * 4u);
  buffer_to_lds<4>(rs, (uint32_t)min(l, valid - 1) * 4u, slot);
}

// A operand rows = tile rows (k = head dim): lane reads chunk c of row r.
__device__ __forceinline__ bf16x8 lds_read_b128(const lds_char* tile, int off) {
  return __builtin_bit_cast(bf16x8, *(const __attribute__((address_space(3))) u32x4*)(tile + off));
}

// Transposing read: for a tile whose rows are the contraction index k and
// whose columns are the MFMA row index m, returns the A operand (m = lane %
// 32) for one 16-row K-step, rows in the order of the accumulator-as-B
// convention above.  Within each 16-lane group, lane i receives element i%4
// of the 8-byte piece addressed by lane 4e + i/4 as its element e; the
// caller's per-lane byte offsets implement that pattern (see tr_offset).
__device__ __forceinline__ bf16x8 lds_read_tr(const lds_char* tile, int off_lo, int off_hi) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off_lo));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off_hi));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  const u32x4 w = {ua[0], ua[1], ub[0], ub[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// Per-lane byte offset of the transposing read covering tile rows
// kbase + 16*ks + {4hh..4hh+3} (rh = 0) or + 8 + {..} (rh = 1) and head-dim
// columns 32*mb + (lane % 32): lane (group g = lane/16, j = lane%16) points
// at row ... + j/4, columns 32*mb + 16*(g%2) + 4*(j%4) .. +3.
template <int D>
__device__ __forceinline__ int tr_offset(int lane, int kbase, int rh, int mb) {
  const int g = lane >> 4, j = lane & 15;
  const int row = kbase + 8 * rh + 4 * (g >> 1) + (j >> 2);
  const int col = 32 * mb + 16 * (g & 1) + 4 * (j & 3);
  return row * (D * 2) + (((col >> 3) ^ swz<D>(row)) << 4) + ((col & 7) << 1);
}

}  // namespace mmsp
