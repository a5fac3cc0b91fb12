// Host-side launch interface between the C-ABI layer (api.hip) and the
// kernel translation units.  Parameters arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmsp {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* q_pos;
  const int32_t* k_pos;
  const int32_t* q_start;  // packed samples: first position of each query's sample, or null
  float* o;
  float* lse;
  int sq, sk, hq, hkv, group, n_qtiles;
  float scale_log2;  // scale * log2(e)
  int causal, accumulate;
  // packed samples: a tile plan (tile_plan.hip) or null; plan_off is the
  // offset of the forward's tile list in it
  const int32_t* plan;
  int plan_off;
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* delta;
  const int32_t* q_pos;
  const int32_t* k_pos;
  const int32_t* q_start;  // packed samples: first position of each query's sample, or null
  float* dq;
  float* dk;
  float* dv;
  int sq, sk, hq, hkv, group, n_ktiles, n_qtiles;
  float scale;
  float scale_log2;
  int causal, accumulate;
  int run_dkdv, run_dq;  // which of the two kernels to enqueue
  // packed samples: a tile plan (tile_plan.hip) or null, with the offsets of
  // the dQ kernel's and the dK/dV kernel's tile lists in it
  const int32_t* plan;
  int plan_dq_off, plan_dkdv_off;
};

// Tile plan of the packed attention kernels: int32 words, a header
// {kPlanMagic, sq, sk, n_fwd, n_dq, n_dkdv, 0, 0}, then three tile lists,
// heaviest tile first (the forward's query tiles, the dQ kernel's query tiles,
// the dK/dV kernel's key tiles), then the work of each tile in the same three
// sections, by tile index.  A kernel uses a plan only when the header names
// its own sq and sk; otherwise it keeps its built-in order.
constexpr int32_t kPlanMagic = 0x4e414c50;
constexpr int kPlanHeader = 8;
struct PlanShape {
  int n_fwd, n_dq, n_dkdv;
  int fwd_off() const { return kPlanHeader; }
  int dq_off() const { return kPlanHeader + n_fwd; }
  int dkdv_off() const { return kPlanHeader + n_fwd + n_dq; }
  int work_off() const { return kPlanHeader + n_fwd + n_dq + n_dkdv; }
  size_t bytes() const { return 4 * (size_t)(kPlanHeader + 2 * (n_fwd + n_dq + n_dkdv)); }
};
PlanShape plan_shape(int sq, int sk);
// plans of n_chunks chunks whose key positions lie sk apart in k_pos, written
// to consecutive plans of PlanShape::bytes() each
hipError_t launch_tile_plan(const int32_t* q_pos, const int32_t* q_start, const int32_t* k_pos,
                            int n_chunks, int sq, int sk, int32_t* plan, hipStream_t stream);

int fwd_rows_per_block();
int fwd_keys_per_tile();
hipError_t launch_attn_fwd(const FwdParams& p, int d, hipStream_t stream);

hipError_t launch_lse_merge(float* o_acc, float* lse_acc, const float* o_part,
                            const float* lse_part, int sq, int hq, int d, uint16_t* o_bf16,
                            hipStream_t stream);

hipError_t launch_bwd_preprocess(const uint16_t* o, const uint16_t* dout, int sq, int hq, int d,
                                 float* delta, float* dq_zero, hipStream_t stream);

int bwd_keys_per_block();
int bwd_rows_per_block();
int dkdv_rows_per_tile();
int dq_keys_per_tile();
hipError_t launch_attn_bwd(const BwdParams& p, int d, hipStream_t stream);

// shard balance: vis/owner scratch of n/g int32 each (MODALITY only)
hipError_t launch_shard_balance(const uint8_t* labels, int n, int n_ranks, int mode, int g,
                                int32_t* perm, int32_t* inv_perm, int32_t* ws_vis,
                                int32_t* ws_owner, hipStream_t stream);

// Allocation-free variant: the device address, on the current device, of the
// library's own static scratch (vis, then owner, kNoallocMaxBlocks int32 each),
// looked up once per device.
constexpr int kNoallocMaxBlocks = 1 << 16;
hipError_t noalloc_balance_scratch(int32_t** vis, int32_t** owner);

// per-sample zigzag of packed samples (starts: n_samples + 1 positions)
hipError_t launch_shard_balance_packed(const int32_t* starts, int n_samples, int n, int n_ranks,
                                       int32_t* perm, int32_t* inv_perm, int32_t* token_start,
                                       hipStream_t stream);

// counts violations of the position preconditions into *count (device)
hipError_t launch_check_positions(const int32_t* pos, const int32_t* starts, int n,
                                  int32_t* count, hipStream_t stream);

// rows of row_bytes moved by an index list: gather dst[i] = src[rows[i]],
// scatter dst[rows[i]] = src[i]; indexed_rows bounds the indexed tensor
hipError_t launch_move_rows(const void* src, const int32_t* rows, int64_t n_rows,
                            int64_t indexed_rows, int64_t row_bytes, void* dst, bool gather,
                            hipStream_t stream);

// rotary embedding of a [s][h][d] bf16 or fp32 tensor (y may equal x)
hipError_t launch_rope(const void* x, void* y, bool bf16, const int32_t* pos, int s, int h, int d,
                       double theta, int inverse, hipStream_t stream);

}  // namespace mmsp
