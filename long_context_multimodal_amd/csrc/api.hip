// C-ABI of libmmsp.so (declared and documented in include/mmsp.h).
//
// Every entry point validates its arguments on the host and returns a
// status before anything is enqueued; it never allocates device memory and
// never synchronises.  Launch errors are reported as MMSP_ERR_HIP.
#include <math.h>

#include "../../include/mmsp.h"
#include "kernels.h"

namespace {

constexpr long long kMaxElems = 0x7fffffffLL;  // element offsets stay in int32 range per row
constexpr int kMaxRanks = 1024;
static_assert(MMSP_NOALLOC_MAX_BLOCKS == mmsp::kNoallocMaxBlocks,
              "header and library agree on the static scratch size");

inline bool bad_dim(int32_t d) { return d != 64 && d != 128; }

inline int check_hip(hipError_t e) { return e == hipSuccess ? MMSP_OK : MMSP_ERR_HIP; }

inline hipStream_t as_stream(hipStream_t s) { return s; }

int check_attn_shapes(int32_t sq, int32_t sk, int32_t hq, int32_t hkv, int32_t d, float scale) {
  if (sq <= 0 || sk <= 0 || hq <= 0 || hkv <= 0) return MMSP_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return MMSP_ERR_SHAPE;
  if (bad_dim(d)) return MMSP_ERR_UNSUPPORTED;
  if (hq % hkv != 0) return MMSP_ERR_DIVISIBILITY;
  if ((long long)sq * hq * d > kMaxElems || (long long)sk * hkv * d > kMaxElems)
    return MMSP_ERR_SHAPE;
  return MMSP_OK;
}

}  // namespace

namespace {

int attn_fwd(const void* q, const void* k, const void* v, const int32_t* q_pos,
             const int32_t* q_start, const int32_t* k_pos, int32_t sq, int32_t sk, int32_t hq,
             int32_t hkv, int32_t d, float scale, uint32_t flags, float* o, float* lse,
             const int32_t* plan, hipStream_t stream) {
  if ((flags & ~(uint32_t)(MMSP_CAUSAL | MMSP_ACCUMULATE)) != 0) return MMSP_ERR_UNSUPPORTED;
  const bool causal = (flags & MMSP_CAUSAL) != 0;
  if (!q || !k || !v || !o || !lse) return MMSP_ERR_NULL;
  if (causal && (!q_pos || !k_pos)) return MMSP_ERR_NULL;
  const int st = check_attn_shapes(sq, sk, hq, hkv, d, scale);
  if (st != MMSP_OK) return st;
  mmsp::FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.q_pos = q_pos;
  p.k_pos = k_pos;
  p.q_start = q_start;
  p.o = o;
  p.lse = lse;
  p.sq = sq;
  p.sk = sk;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  const int bm = mmsp::fwd_rows_per_block();
  p.n_qtiles = (sq + bm - 1) / bm;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal = causal ? 1 : 0;
  p.accumulate = (flags & MMSP_ACCUMULATE) ? 1 : 0;
  p.plan = plan;
  p.plan_off = mmsp::plan_shape(sq, sk).fwd_off();
  return check_hip(mmsp::launch_attn_fwd(p, d, as_stream(stream)));
}

int attn_bwd(const void* q, const void* k, const void* v, const void* dout, const float* lse,
             const float* delta, const int32_t* q_pos, const int32_t* q_start,
             const int32_t* k_pos, int32_t sq, int32_t sk, int32_t hq, int32_t hkv, int32_t d,
             float scale, uint32_t flags, float* dq_acc, float* dk, float* dv, const int32_t* plan,
             hipStream_t stream) {
  if ((flags & ~(uint32_t)(MMSP_CAUSAL | MMSP_ACCUMULATE | MMSP_BWD_NO_DQ | MMSP_BWD_NO_DKDV)) !=
      0)
    return MMSP_ERR_UNSUPPORTED;
  const bool run_dq = (flags & MMSP_BWD_NO_DQ) == 0;
  const bool run_dkdv = (flags & MMSP_BWD_NO_DKDV) == 0;
  if (!run_dq && !run_dkdv) return MMSP_ERR_UNSUPPORTED;
  const bool causal = (flags & MMSP_CAUSAL) != 0;
  if (!q || !k || !v || !dout || !lse || !delta) return MMSP_ERR_NULL;
  if ((run_dq && !dq_acc) || (run_dkdv && (!dk || !dv))) return MMSP_ERR_NULL;
  if (causal && (!q_pos || !k_pos)) return MMSP_ERR_NULL;
  const int st = check_attn_shapes(sq, sk, hq, hkv, d, scale);
  if (st != MMSP_OK) return st;
  mmsp::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.delta = delta;
  p.q_pos = q_pos;
  p.k_pos = k_pos;
  p.q_start = q_start;
  p.dq = dq_acc;
  p.dk = dk;
  p.dv = dv;
  p.sq = sq;
  p.sk = sk;
  p.hq = hq;
  p.hkv = hkv;
  p.group = hq / hkv;
  const int bk = mmsp::bwd_keys_per_block();
  const int bq = mmsp::bwd_rows_per_block();
  p.n_ktiles = (sk + bk - 1) / bk;
  p.n_qtiles = (sq + bq - 1) / bq;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal = causal ? 1 : 0;
  p.accumulate = (flags & MMSP_ACCUMULATE) ? 1 : 0;
  p.run_dkdv = run_dkdv ? 1 : 0;
  p.run_dq = run_dq ? 1 : 0;
  const mmsp::PlanShape ps = mmsp::plan_shape(sq, sk);
  p.plan = plan;
  p.plan_dq_off = ps.dq_off();
  p.plan_dkdv_off = ps.dkdv_off();
  return check_hip(mmsp::launch_attn_bwd(p, d, as_stream(stream)));
}

// A tile plan given to a packed call must be as large as its sizes need.
int check_plan(const void* plan, size_t plan_bytes, int32_t sq, int32_t sk) {
  if (plan == nullptr) return MMSP_OK;
  if (sq <= 0 || sk <= 0) return MMSP_ERR_SHAPE;
  return plan_bytes < mmsp::plan_shape(sq, sk).bytes() ? MMSP_ERR_WORKSPACE : MMSP_OK;
}

}  // namespace

extern "C" {

const char* mmsp_status_string(int status) {
  switch (status) {
    case MMSP_OK: return "ok";
    case MMSP_ERR_NULL: return "a required pointer is NULL";
    case MMSP_ERR_SHAPE: return "invalid size or scale";
    case MMSP_ERR_UNSUPPORTED: return "unsupported head_dim, mode or flag";
    case MMSP_ERR_DIVISIBILITY: return "divisibility requirement not met";
    case MMSP_ERR_WORKSPACE: return "workspace missing or too small";
    case MMSP_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int mmsp_abi_version(void) { return MMSP_ABI_VERSION; }

int mmsp_device_info(int32_t device, int32_t* compute_units, int32_t* peak_clock_khz,
                     int32_t* l2_bytes) {
  if (!compute_units || !peak_clock_khz || !l2_bytes) return MMSP_ERR_NULL;
  int cu = 0, clk = 0, l2 = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      hipDeviceGetAttribute(&clk, hipDeviceAttributeClockRate, device) != hipSuccess ||
      hipDeviceGetAttribute(&l2, hipDeviceAttributeL2CacheSize, device) != hipSuccess)
    return MMSP_ERR_HIP;
  *compute_units = cu;
  *peak_clock_khz = clk;
  *l2_bytes = l2;
  return MMSP_OK;
}

size_t mmsp_shard_balance_workspace_bytes(int64_t n, int32_t n_ranks, int32_t mode,
                                          int32_t granularity) {
  (void)n_ranks;
  if (mode != MMSP_BALANCE_MODALITY || n <= 0 || granularity <= 0) return 0;
  const int64_t n_blocks = n / granularity;
  return (size_t)(2 * n_blocks) * sizeof(int32_t);
}

namespace {
// host checks shared by the two shard-balance entry points
int check_balance(const uint8_t* d_labels, int64_t n, int32_t n_ranks, int32_t mode,
                  int32_t granularity, const int32_t* d_perm) {
  if (mode != MMSP_BALANCE_ZIGZAG && mode != MMSP_BALANCE_MODALITY) return MMSP_ERR_UNSUPPORTED;
  if (d_perm == nullptr) return MMSP_ERR_NULL;
  if (mode == MMSP_BALANCE_MODALITY && d_labels == nullptr) return MMSP_ERR_NULL;
  if (n <= 0 || n > kMaxElems || n_ranks <= 0 || n_ranks > kMaxRanks) return MMSP_ERR_SHAPE;
  if (mode == MMSP_BALANCE_ZIGZAG) {
    if (n % (2LL * n_ranks) != 0) return MMSP_ERR_DIVISIBILITY;
  } else {
    if (granularity <= 0) return MMSP_ERR_SHAPE;
    if (n % (2LL * n_ranks * granularity) != 0) return MMSP_ERR_DIVISIBILITY;
  }
  return MMSP_OK;
}
}  // namespace

int mmsp_shard_balance(const uint8_t* d_labels, int64_t n, int32_t n_ranks, int32_t mode,
                       int32_t granularity, int32_t* d_perm, int32_t* d_inv_perm,
                       void* d_workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_balance(d_labels, n, n_ranks, mode, granularity, d_perm);
  if (st != MMSP_OK) return st;
  int32_t* ws_vis = nullptr;
  int32_t* ws_owner = nullptr;
  if (mode == MMSP_BALANCE_MODALITY) {
    const size_t need = mmsp_shard_balance_workspace_bytes(n, n_ranks, mode, granularity);
    if (d_workspace == nullptr || workspace_bytes < need) return MMSP_ERR_WORKSPACE;
    ws_vis = static_cast<int32_t*>(d_workspace);
    ws_owner = ws_vis + n / granularity;
  }
  return check_hip(mmsp::launch_shard_balance(d_labels, (int)n, n_ranks, mode, granularity,
                                              d_perm, d_inv_perm, ws_vis, ws_owner,
                                              as_stream(stream)));
}

int mmsp_shard_balance_noalloc(const uint8_t* d_labels, int64_t n, int32_t n_ranks, int32_t mode,
                               int32_t granularity, int32_t* d_perm, int32_t* d_inv_perm,
                               hipStream_t stream) {
  const int st = check_balance(d_labels, n, n_ranks, mode, granularity, d_perm);
  if (st != MMSP_OK) return st;
  int32_t* ws_vis = nullptr;
  int32_t* ws_owner = nullptr;
  if (mode == MMSP_BALANCE_MODALITY) {
    if (n / granularity > MMSP_NOALLOC_MAX_BLOCKS) return MMSP_ERR_WORKSPACE;
    if (mmsp::noalloc_balance_scratch(&ws_vis, &ws_owner) != hipSuccess) return MMSP_ERR_HIP;
  }
  return check_hip(mmsp::launch_shard_balance(d_labels, (int)n, n_ranks, mode, granularity,
                                              d_perm, d_inv_perm, ws_vis, ws_owner,
                                              as_stream(stream)));
}

int mmsp_shard_balance_packed(const int32_t* d_starts, int32_t n_samples, int64_t n,
                              int32_t n_ranks, int32_t* d_perm, int32_t* d_inv_perm,
                              int32_t* d_token_start, hipStream_t stream) {
  if (!d_starts || !d_perm) return MMSP_ERR_NULL;
  if (n <= 0 || n > kMaxElems || n_ranks <= 0 || n_ranks > kMaxRanks || n_samples <= 0 ||
      n_samples > n)
    return MMSP_ERR_SHAPE;
  if (n % (2LL * n_ranks) != 0) return MMSP_ERR_DIVISIBILITY;
  return check_hip(mmsp::launch_shard_balance_packed(d_starts, n_samples, (int)n, n_ranks,
                                                     d_perm, d_inv_perm, d_token_start,
                                                     as_stream(stream)));
}

namespace {
int move_rows(const void* src, const int32_t* rows, int64_t n_rows, int64_t indexed_rows,
              int64_t row_bytes, void* dst, bool gather, hipStream_t stream) {
  if (!src || !rows || !dst) return MMSP_ERR_NULL;
  if (n_rows <= 0 || indexed_rows <= 0 || n_rows > kMaxElems || indexed_rows > kMaxElems ||
      row_bytes < 16 || row_bytes % 16 != 0 || row_bytes / 16 > kMaxElems)
    return MMSP_ERR_SHAPE;
  return check_hip(mmsp::launch_move_rows(src, rows, n_rows, indexed_rows, row_bytes, dst, gather,
                                          as_stream(stream)));
}
}  // namespace

int mmsp_check_positions(const int32_t* d_pos, const int32_t* d_starts, int32_t n,
                         int32_t* d_violations, hipStream_t stream) {
  if (!d_pos || !d_violations) return MMSP_ERR_NULL;
  if (n <= 0) return MMSP_ERR_SHAPE;
  return check_hip(mmsp::launch_check_positions(d_pos, d_starts, n, d_violations,
                                                as_stream(stream)));
}

int mmsp_shard_gather(const void* d_src, int64_t src_rows, const int32_t* d_rows, int64_t n_rows,
                      int64_t row_bytes, void* d_dst, hipStream_t stream) {
  return move_rows(d_src, d_rows, n_rows, src_rows, row_bytes, d_dst, true, stream);
}

int mmsp_shard_scatter(const void* d_src, int64_t n_rows, const int32_t* d_rows,
                       int64_t dst_rows, int64_t row_bytes, void* d_dst, hipStream_t stream) {
  return move_rows(d_src, d_rows, n_rows, dst_rows, row_bytes, d_dst, false, stream);
}

int mmsp_attn_fwd_chunk(const void* q, const void* k, const void* v, const int32_t* q_pos,
                        const int32_t* k_pos, int32_t sq, int32_t sk, int32_t hq, int32_t hkv,
                        int32_t d, float scale, uint32_t flags, float* o, float* lse,
                        hipStream_t stream) {
  return attn_fwd(q, k, v, q_pos, nullptr, k_pos, sq, sk, hq, hkv, d, scale, flags, o, lse,
                  nullptr, stream);
}

int mmsp_attn_fwd_chunk_packed(const void* q, const void* k, const void* v,
                               const int32_t* q_pos, const int32_t* q_start,
                               const int32_t* k_pos, const void* plan, size_t plan_bytes,
                               int32_t sq, int32_t sk, int32_t hq, int32_t hkv, int32_t d,
                               float scale, uint32_t flags, float* o, float* lse,
                               hipStream_t stream) {
  if (!(flags & MMSP_CAUSAL)) return MMSP_ERR_UNSUPPORTED;
  if (!q_start) return MMSP_ERR_NULL;
  const int st = check_plan(plan, plan_bytes, sq, sk);
  if (st != MMSP_OK) return st;
  return attn_fwd(q, k, v, q_pos, q_start, k_pos, sq, sk, hq, hkv, d, scale, flags, o, lse,
                  static_cast<const int32_t*>(plan), stream);
}

size_t mmsp_attn_packed_plan_bytes(int32_t sq, int32_t sk) {
  if (sq <= 0 || sk <= 0) return 0;
  return mmsp::plan_shape(sq, sk).bytes();
}

int mmsp_attn_packed_plan(const int32_t* q_pos, const int32_t* q_start, const int32_t* k_pos,
                          int32_t sq, int32_t sk, void* plan, size_t plan_bytes,
                          hipStream_t stream) {
  return mmsp_attn_packed_plans(q_pos, q_start, k_pos, 1, sq, sk, plan, plan_bytes, stream);
}

int mmsp_attn_packed_plans(const int32_t* q_pos, const int32_t* q_start, const int32_t* k_pos,
                           int32_t n_chunks, int32_t sq, int32_t sk, void* plans,
                           size_t plans_bytes, hipStream_t stream) {
  if (!q_pos || !q_start || !k_pos || !plans) return MMSP_ERR_NULL;
  if (sq <= 0 || sk <= 0 || n_chunks <= 0 || n_chunks > kMaxRanks) return MMSP_ERR_SHAPE;
  if ((long long)n_chunks * sk > kMaxElems) return MMSP_ERR_SHAPE;
  if (plans_bytes / (size_t)n_chunks < mmsp::plan_shape(sq, sk).bytes()) return MMSP_ERR_WORKSPACE;
  return check_hip(mmsp::launch_tile_plan(q_pos, q_start, k_pos, n_chunks, sq, sk,
                                          static_cast<int32_t*>(plans), as_stream(stream)));
}

int mmsp_lse_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                   int32_t sq, int32_t hq, int32_t d, void* o_final_bf16, hipStream_t stream) {
  if (!o_acc || !lse_acc) return MMSP_ERR_NULL;
  if ((o_part == nullptr) != (lse_part == nullptr)) return MMSP_ERR_NULL;
  if (sq <= 0 || hq <= 0) return MMSP_ERR_SHAPE;
  if (bad_dim(d)) return MMSP_ERR_UNSUPPORTED;
  if ((long long)sq * hq * d > kMaxElems) return MMSP_ERR_SHAPE;
  if (o_part == nullptr && o_final_bf16 == nullptr) return MMSP_OK;  // nothing to do
  return check_hip(mmsp::launch_lse_merge(o_acc, lse_acc, o_part, lse_part, sq, hq, d,
                                          static_cast<uint16_t*>(o_final_bf16),
                                          as_stream(stream)));
}

int mmsp_attn_bwd_preprocess(const void* o, const void* dout, int32_t sq, int32_t hq, int32_t d,
                             float* delta, float* dq_zero, hipStream_t stream) {
  if (!o || !dout || !delta) return MMSP_ERR_NULL;
  if (sq <= 0 || hq <= 0) return MMSP_ERR_SHAPE;
  if (bad_dim(d)) return MMSP_ERR_UNSUPPORTED;
  if ((long long)sq * hq * d > kMaxElems) return MMSP_ERR_SHAPE;
  return check_hip(mmsp::launch_bwd_preprocess(static_cast<const uint16_t*>(o),
                                               static_cast<const uint16_t*>(dout), sq, hq, d,
                                               delta, dq_zero, as_stream(stream)));
}

int mmsp_attn_bwd_chunk(const void* q, const void* k, const void* v, const void* dout,
                        const float* lse, const float* delta, const int32_t* q_pos,
                        const int32_t* k_pos, int32_t sq, int32_t sk, int32_t hq, int32_t hkv,
                        int32_t d, float scale, uint32_t flags, float* dq_acc, float* dk,
                        float* dv, hipStream_t stream) {
  return attn_bwd(q, k, v, dout, lse, delta, q_pos, nullptr, k_pos, sq, sk, hq, hkv, d, scale,
                  flags, dq_acc, dk, dv, nullptr, stream);
}

int mmsp_attn_bwd_chunk_packed(const void* q, const void* k, const void* v, const void* dout,
                               const float* lse, const float* delta, const int32_t* q_pos,
                               const int32_t* q_start, const int32_t* k_pos, const void* plan,
                               size_t plan_bytes, int32_t sq, int32_t sk, int32_t hq,
                               int32_t hkv, int32_t d, float scale, uint32_t flags,
                               float* dq_acc, float* dk, float* dv, hipStream_t stream) {
  if (!(flags & MMSP_CAUSAL)) return MMSP_ERR_UNSUPPORTED;
  if (!q_start) return MMSP_ERR_NULL;
  const int st = check_plan(plan, plan_bytes, sq, sk);
  if (st != MMSP_OK) return st;
  return attn_bwd(q, k, v, dout, lse, delta, q_pos, q_start, k_pos, sq, sk, hq, hkv, d, scale,
                  flags, dq_acc, dk, dv, static_cast<const int32_t*>(plan), stream);
}

// One rank's ring loop: chunk (rank - t) mod n_chunks at step t.  Every
// argument of every chunk is checked before the first launch.
int mmsp_ring_forward(const void* q, const void* const* k_chunks, const void* const* v_chunks,
                      const int32_t* q_pos, const int32_t* const* k_pos_chunks,
                      const int32_t* q_start, int32_t n_chunks, int32_t rank, int32_t sq,
                      int32_t sk, int32_t hq, int32_t hkv, int32_t d, float scale,
                      uint32_t flags, float* o, float* lse, void* o_final_bf16, hipStream_t stream) {
  if ((flags & ~(uint32_t)MMSP_CAUSAL) != 0) return MMSP_ERR_UNSUPPORTED;
  const bool causal = (flags & MMSP_CAUSAL) != 0;
  if (q_start && !causal) return MMSP_ERR_UNSUPPORTED;
  if (!k_chunks || !v_chunks || (causal && !k_pos_chunks)) return MMSP_ERR_NULL;
  if (n_chunks <= 0 || rank < 0 || rank >= n_chunks) return MMSP_ERR_SHAPE;
  if (!q || !o || !lse || (causal && !q_pos)) return MMSP_ERR_NULL;
  for (int c = 0; c < n_chunks; ++c)
    if (!k_chunks[c] || !v_chunks[c] || (causal && !k_pos_chunks[c])) return MMSP_ERR_NULL;
  int st = check_attn_shapes(sq, sk, hq, hkv, d, scale);
  if (st != MMSP_OK) return st;
  for (int t = 0; t < n_chunks; ++t) {
    const int c = ((rank - t) % n_chunks + n_chunks) % n_chunks;
    const uint32_t f = flags | (t > 0 ? (uint32_t)MMSP_ACCUMULATE : 0u);
    st = attn_fwd(q, k_chunks[c], v_chunks[c], q_pos, q_start, causal ? k_pos_chunks[c] : nullptr,
                  sq, sk, hq, hkv, d, scale, f, o, lse, nullptr, stream);
    if (st != MMSP_OK) return st;
  }
  if (o_final_bf16 == nullptr) return MMSP_OK;
  return check_hip(mmsp::launch_lse_merge(o, lse, nullptr, nullptr, sq, hq, d,
                                          static_cast<uint16_t*>(o_final_bf16),
                                          as_stream(stream)));
}

int mmsp_ring_backward(const void* q, const void* const* k_chunks, const void* const* v_chunks,
                       const void* dout, const void* o_bf16, const float* lse,
                       const int32_t* q_pos, const int32_t* const* k_pos_chunks,
                       const int32_t* q_start, int32_t n_chunks, int32_t rank, int32_t sq,
                       int32_t sk, int32_t hq, int32_t hkv, int32_t d, float scale,
                       uint32_t flags, float* delta, float* dq, float* const* dk_chunks,
                       float* const* dv_chunks, hipStream_t stream) {
  if ((flags & ~(uint32_t)(MMSP_CAUSAL | MMSP_ACCUMULATE)) != 0) return MMSP_ERR_UNSUPPORTED;
  const bool causal = (flags & MMSP_CAUSAL) != 0;
  if (q_start && !causal) return MMSP_ERR_UNSUPPORTED;
  if (!k_chunks || !v_chunks || !dk_chunks || !dv_chunks || (causal && !k_pos_chunks))
    return MMSP_ERR_NULL;
  if (n_chunks <= 0 || rank < 0 || rank >= n_chunks) return MMSP_ERR_SHAPE;
  if (!q || !dout || !o_bf16 || !lse || !delta || !dq || (causal && !q_pos)) return MMSP_ERR_NULL;
  for (int c = 0; c < n_chunks; ++c)
    if (!k_chunks[c] || !v_chunks[c] || !dk_chunks[c] || !dv_chunks[c] ||
        (causal && !k_pos_chunks[c]))
      return MMSP_ERR_NULL;
  int st = check_attn_shapes(sq, sk, hq, hkv, d, scale);
  if (st != MMSP_OK) return st;
  // delta from the bf16 output; dq zeroed in the same pass
  st = check_hip(mmsp::launch_bwd_preprocess(static_cast<const uint16_t*>(o_bf16),
                                             static_cast<const uint16_t*>(dout), sq, hq, d, delta,
                                             dq, as_stream(stream)));
  if (st != MMSP_OK) return st;
  for (int t = 0; t < n_chunks; ++t) {
    const int c = ((rank - t) % n_chunks + n_chunks) % n_chunks;
    st = attn_bwd(q, k_chunks[c], v_chunks[c], dout, lse, delta, q_pos, q_start,
                  causal ? k_pos_chunks[c] : nullptr, sq, sk, hq, hkv, d, scale, flags, dq,
                  dk_chunks[c], dv_chunks[c], nullptr, stream);
    if (st != MMSP_OK) return st;
  }
  return MMSP_OK;
}

int mmsp_rope(const void* x, void* y, int32_t dtype, const int32_t* pos, int32_t s, int32_t h,
              int32_t d, double theta, int32_t inverse, hipStream_t stream) {
  if (!x || !y || !pos) return MMSP_ERR_NULL;
  if (dtype != MMSP_DTYPE_BF16 && dtype != MMSP_DTYPE_F32) return MMSP_ERR_UNSUPPORTED;
  if (inverse != 0 && inverse != 1) return MMSP_ERR_UNSUPPORTED;
  if (bad_dim(d)) return MMSP_ERR_UNSUPPORTED;
  if (s <= 0 || h <= 0 || (long long)s * h * d > kMaxElems) return MMSP_ERR_SHAPE;
  if (!(theta > 1.0) || !isfinite(theta)) return MMSP_ERR_SHAPE;
  return check_hip(mmsp::launch_rope(x, y, dtype == MMSP_DTYPE_BF16, pos, s, h, d, theta, inverse,
                                     as_stream(stream)));
}

}  // extern "C"
