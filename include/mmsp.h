/*
 * mmsp.h -- C-ABI of libmmsp.so: one rank's share of multi-modal sequence-
 * parallel (MM-SP) causal attention on an AMD MI355X (gfx950).
 *
 * What is computed (sources are web pages, cited by title and section):
 *
 *  - "LongVILA Guide: 2M Context Multi-Modal AI Model", section
 *    "Multi-Modal Sequence Parallelism (MM-SP) Mechanics": each rank holds
 *    N/P tokens; K/V chunks travel around a ring and every ring step runs one
 *    attention kernel of the local queries against the chunk that arrived.
 *  - Same page, section "Implementation: PyTorch Distributed Pipeline and
 *    Token Routing": the per-step body scales the query-key dot products by
 *    1/sqrt(head_dim), applies a softmax and accumulates the weighted values
 *    into an output accumulator, one chunk per step.
 *  - Same page, section "Problem", item 2, and "Ultra-Large Multimodal LLM
 *    Inference ...", section 4 "Load Balancing for Tensor Parallelism":
 *    modality-dense and text-only regions give ranks unequal work; work is
 *    dispatched by modality token density.
 *  - "LongVILA - ... (Jason's Study)", section "What it is": training at 2M
 *    tokens runs without gradient checkpointing, so the backward consumes
 *    the saved forward statistics.
 *
 * Conventions shared by every entry point:
 *
 *  - Every data pointer is a DEVICE pointer owned by the caller; the library
 *    keeps no pointer after the call returns and allocates no device memory
 *    (scratch comes from the caller, sized by a *_workspace_bytes query; the
 *    one exception, mmsp_shard_balance_noalloc, uses a static array of the
 *    library's code object instead).
 *  - bf16 tensors are passed as `const void*` holding IEEE bfloat16 bits.
 *    Layouts are row-major and contiguous: token-major activations
 *    [tokens][heads][head_dim]; per-head statistics [heads][tokens].
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it and returns; device faults surface at the caller's
 *    next synchronisation of that stream.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    nonzero return means nothing was launched.  Calls are thread-safe and
 *    keep no global device state (but for that static array).  Position
 *    arrays must be strictly increasing (a precondition, not checked).
 *  - No entry point allocates, synchronises or enqueues a memset (buffers
 *    that must start at zero are cleared by the library's own kernels), so
 *    the enqueued work can be captured in a HIP graph; the host-only
 *    queries (status strings, version, device info, workspace size) launch
 *    nothing.
 */
#ifndef MMSP_H
#define MMSP_H

#include <stddef.h>
#include <stdint.h>

/* The HIP runtime's stream handle (the same declaration as hip_runtime_api.h,
 * so this header needs no HIP include and agrees with it when both are seen). */
typedef struct ihipStream_t* hipStream_t;

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status ------------------------------------------------------------ */
enum {
  MMSP_OK = 0,
  MMSP_ERR_NULL = -1,         /* a required pointer is NULL                 */
  MMSP_ERR_SHAPE = -2,        /* a size is <= 0, too large, or scale <= 0   */
  MMSP_ERR_UNSUPPORTED = -3,  /* head_dim not in {64,128}; unknown mode/flag*/
  MMSP_ERR_DIVISIBILITY = -4, /* hq % hkv != 0; n not divisible by 2*P*g    */
  MMSP_ERR_WORKSPACE = -5,    /* workspace NULL or smaller than required    */
  MMSP_ERR_HIP = -6           /* the HIP runtime reported a launch error    */
};

/* Static string naming a status code ("unknown status" for others). */
const char* mmsp_status_string(int status);

/* Version of this ABI; bumped on any incompatible change. */
int mmsp_abi_version(void);
#define MMSP_ABI_VERSION 1

/* Compute units, peak shader clock (kHz) and L2 size (bytes, per XCD on a
 * multi-die part) of a device, as the HIP runtime reports them; used to state
 * the clock a measurement could reach.  Host-only query, no launch. */
int mmsp_device_info(int32_t device, int32_t* compute_units, int32_t* peak_clock_khz,
                     int32_t* l2_bytes);

/* ---- a1: shard balance ---------------------------------------------------
 * Permutation of an n-token stream into n_ranks shards of equal causal work
 * (query position p attends to p+1 keys).  Problem statement: "LongVILA
 * Guide ...", section "Problem", item 2; remedy by modality token density:
 * "Ultra-Large Multimodal LLM Inference ...", section 4.
 *
 * MMSP_BALANCE_ZIGZAG: requires n % (2*n_ranks) == 0, L = n/(2*n_ranks);
 *   rank r owns positions [r*L,(r+1)*L) then [(2P-1-r)*L,(2P-r)*L).
 *   `d_labels` may be NULL; `granularity` is ignored.
 * MMSP_BALANCE_MODALITY: requires n % (2*n_ranks*granularity) == 0.  Blocks
 *   of `granularity` tokens; each round of 2P consecutive blocks is paired
 *   outside-in (pair a = blocks 2jP+a and 2jP+2P-1-a); pairs in order of
 *   decreasing visual count (ties: smaller a) go to ranks in order of
 *   increasing running visual total (ties: smaller rank).  `d_labels` is
 *   uint8[n], 0 = text, nonzero = visual.
 *
 * Output: d_perm int32[n], rank-major: rank r's positions are
 * d_perm[r*n/P .. (r+1)*n/P), ascending.  d_inv_perm (nullable) int32[n]
 * with d_inv_perm[d_perm[i]] = i.  1 <= n_ranks <= 1024, n <= 2^31-1.
 * The result is an integer function of the labels: bit-exact and unique.
 */
enum { MMSP_BALANCE_ZIGZAG = 0, MMSP_BALANCE_MODALITY = 1 };

size_t mmsp_shard_balance_workspace_bytes(int64_t n, int32_t n_ranks, int32_t mode,
                                          int32_t granularity);
int mmsp_shard_balance(const uint8_t* d_labels, int64_t n, int32_t n_ranks, int32_t mode,
                       int32_t granularity, int32_t* d_perm, int32_t* d_inv_perm,
                       void* d_workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- a1 without allocation ---------------------------------------------------
 * For callers that cannot allocate device memory or hand over a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same permutation as mmsp_shard_balance, bit for bit, with
 * MODALITY's scratch taken from an array the library holds in each device's
 * memory (2 * MMSP_NOALLOC_MAX_BLOCKS int32, 512 KiB, kept until the process
 * ends).  Arguments and checks are those of mmsp_shard_balance, less the
 * workspace; MODALITY with n / granularity > MMSP_NOALLOC_MAX_BLOCKS returns
 * MMSP_ERR_WORKSPACE.  The current device must be the stream's device: the
 * array's address is looked up (hipGetSymbolAddress) on the first call on
 * each device; MMSP_ERR_HIP if that fails.  Calls on one device share the
 * array, so two calls whose work may overlap on that device (two streams,
 * two threads) race; calls ordered on one stream do not.  Nothing in the
 * array needs to start at zero: every call writes what it reads.
 */
#define MMSP_NOALLOC_MAX_BLOCKS 65536
int mmsp_shard_balance_noalloc(const uint8_t* d_labels, int64_t n, int32_t n_ranks, int32_t mode,
                               int32_t granularity, int32_t* d_perm, int32_t* d_inv_perm,
                               hipStream_t stream);

/* ---- a1 for packed samples: per-sample zigzag ------------------------------
 * Variable-length videos packed into one buffer with reset attention masks
 * ("LongVILA Guide ...", sections "Three-Stage Long-Context Alignment
 * Curriculum", stage 3, and "Critical Operational Best Practices").  A query
 * sees only keys of its own sample, so each sample is zigzagged on its own:
 * sample s = positions [starts[s], starts[s+1]), length a positive multiple
 * of 2*n_ranks, L_s = length/(2*n_ranks); rank r takes its blocks r and
 * 2P-1-r.  Every rank then holds 2*L_s tokens and exactly equal causal work
 * of every sample.
 *
 * d_starts      int32 [n_samples + 1] (device): 0 = starts[0] < ... <
 *               starts[n_samples] = n.
 * d_perm        int32 [n], rank-major: rank r's positions are
 *               d_perm[r*n/P .. (r+1)*n/P), sample by sample, ascending.
 * d_inv_perm    (nullable) int32 [n], d_inv_perm[d_perm[i]] = i.
 * d_token_start (nullable) int32 [n]: starts[s] of the sample of the token
 *               in slot i -- the q_start array of the *_packed attention
 *               calls for any rank's shard.
 * Host checks: n % (2*n_ranks) == 0, 1 <= n_samples <= n.  The sample
 * boundaries live on the device and are not checked on the host: every slot
 * is first set to -1 and tokens of a sample whose boundaries are not
 * multiples of 2*n_ranks inside [0, n] are left unplaced (their slots keep
 * -1).  Bit-exact integer result.
 */
int mmsp_shard_balance_packed(const int32_t* d_starts, int32_t n_samples, int64_t n,
                              int32_t n_ranks, int32_t* d_perm, int32_t* d_inv_perm,
                              int32_t* d_token_start, hipStream_t stream);

/* ---- precondition check of positions ----------------------------------------
 * The attention calls take position arrays as strictly increasing and packed
 * sample starts as non-decreasing, non-negative and not after their
 * position, without checking (a precondition: a violation gives wrong
 * results, never an out-of-bounds access).  This call counts, on the device,
 * the indices i that break them: pos[i] <= pos[i-1]; with d_starts (nullable)
 * also d_starts[i] > pos[i] or < 0, and d_starts[i] < d_starts[i-1].  The
 * count is written to d_violations (one device int32; the call zeroes it
 * first with a kernel).  n >= 1.  For debugging; the Python binding runs it
 * before every attention call when MMSP_CHECK_POSITIONS=1.
 */
int mmsp_check_positions(const int32_t* d_pos, const int32_t* d_starts, int32_t n,
                         int32_t* d_violations, hipStream_t stream);

/* ---- a1: token rows into shard order, and back -----------------------------
 * Each rank holds N/P tokens of the stream ("LongVILA Guide ...", section
 * "Multi-Modal Sequence Parallelism (MM-SP) Mechanics"); under a balance
 * permutation those are the rows its d_perm slice names (mmsp_shard_balance
 * or mmsp_shard_balance_packed), moved here from token order.
 * Gather:  dst[i] = src[rows[i]]  for i < n_rows  (rows[i] outside
 *          [0, src_rows) gives a zero row, e.g. the -1 slots of unplaced
 *          packed samples).
 * Scatter: dst[rows[i]] = src[i]  for i < n_rows  (rows[i] outside
 *          [0, dst_rows) is skipped); rows must be distinct, or writes race.
 * A row is row_bytes contiguous bytes (a multiple of 16, e.g. heads * d * 2
 * for bf16 activations); src and dst must not overlap.  n_rows, src_rows /
 * dst_rows >= 1 and < 2^31 (else MMSP_ERR_SHAPE).  Bit-exact byte copy,
 * memory-bound.
 */
int mmsp_shard_gather(const void* d_src, int64_t src_rows, const int32_t* d_rows, int64_t n_rows,
                      int64_t row_bytes, void* d_dst, hipStream_t stream);
int mmsp_shard_scatter(const void* d_src, int64_t n_rows, const int32_t* d_rows,
                       int64_t dst_rows, int64_t row_bytes, void* d_dst, hipStream_t stream);

/* ---- a2: attention of the query shard against one KV chunk ---------------
 * Source: "LongVILA Guide ...", sections "Multi-Modal Sequence Parallelism
 * (MM-SP) Mechanics" (one attention kernel per ring step on the current KV
 * chunk) and "Implementation ..." (scores = q.k * scale, softmax, weighted
 * sum of V).
 *
 * q      bf16 [sq][hq][d]          k, v   bf16 [sk][hkv][d]
 * q_pos  int32 [sq], k_pos int32 [sk]: global token positions, strictly
 *        increasing; with MMSP_CAUSAL key j is visible to query i iff
 *        k_pos[j] <= q_pos[i] (may be NULL without MMSP_CAUSAL: all visible).
 * scale  > 0; the usual value is 1/sqrt(d).
 * GQA    query head h reads KV head h / (hq/hkv); requires hq % hkv == 0.
 * o      fp32 [sq][hq][d]; lse fp32 [hq][sq] (natural log of the sum of
 *        exp(scale*q.k) over the visible keys of this chunk).
 * flags  MMSP_CAUSAL | MMSP_ACCUMULATE.  Without ACCUMULATE, (o, lse) are
 *        overwritten with this chunk's normalised result; a row with no
 *        visible key gets o = 0, lse = -inf.  With ACCUMULATE, (o, lse) hold a
 *        running result over earlier chunks (start from o = 0, lse = -inf)
 *        and are merged in place with this chunk's result exactly as
 *        mmsp_lse_merge does; rows with no visible key are left untouched.
 * d in {64, 128}; sq, sk >= 1; hq*sq*d and hkv*sk*d < 2^31.
 */
enum { MMSP_CAUSAL = 1u, MMSP_ACCUMULATE = 2u };

int mmsp_attn_fwd_chunk(const void* q, const void* k, const void* v, const int32_t* q_pos,
                        const int32_t* k_pos, int32_t sq, int32_t sk, int32_t hq, int32_t hkv,
                        int32_t d, float scale, uint32_t flags, float* o, float* lse,
                        hipStream_t stream);

/* ---- a2 with packed samples -------------------------------------------------
 * As mmsp_attn_fwd_chunk, with reset attention masks between packed samples
 * ("LongVILA Guide ...", "Critical Operational Best Practices"): a query
 * sees only keys of its own sample.  Samples are contiguous position ranges,
 * so that is q_start[i] <= k_pos[j] <= q_pos[i].
 * q_start int32 [sq] (device, required): first position of query i's sample,
 *         q_start[i] <= q_pos[i], non-decreasing in i (as mmsp_shard_balance_
 *         packed produces it).  flags must include MMSP_CAUSAL.
 * plan    (nullable) tile plan from mmsp_attn_packed_plan for these
 *         positions, plan_bytes its size (below); NULL: built-in tile order.
 */
int mmsp_attn_fwd_chunk_packed(const void* q, const void* k, const void* v,
                               const int32_t* q_pos, const int32_t* q_start,
                               const int32_t* k_pos, const void* plan, size_t plan_bytes,
                               int32_t sq, int32_t sk, int32_t hq, int32_t hkv, int32_t d,
                               float scale, uint32_t flags, float* o, float* lse,
                               hipStream_t stream);

/* ---- tile plan of the packed attention calls --------------------------------
 * Scheduling only, not part of the method: the results of the packed calls
 * are the same bit for bit with or without a plan.  With packed samples
 * ("LongVILA Guide ...", "Critical Operational Best Practices") the work of
 * a workgroup depends on the samples its tile holds, and the built-in tile
 * order (made for the plain causal shard) can leave the heaviest tiles to the
 * end of the launch.  mmsp_attn_packed_plan counts each tile's work from the
 * positions and lists the tiles heaviest first for the forward, the dQ and
 * the dK/dV kernels; passed as `plan` to mmsp_attn_fwd_chunk_packed and
 * mmsp_attn_bwd_chunk_packed, the kernels take their tiles in that order.
 * One plan serves the forward and the backward of the same (q_pos, q_start,
 * k_pos).
 *
 * plan        device buffer of plan_bytes >= mmsp_attn_packed_plan_bytes(sq,
 *             sk) bytes (32 + 8 * (ceil(sq/256) + ceil(sq/128) + ceil(sk/128))),
 *             owned by the caller; written by mmsp_attn_packed_plan on
 *             `stream`.  NULL in the attention calls keeps the built-in order.
 * q_pos, q_start, k_pos as in mmsp_attn_fwd_chunk_packed; sq, sk >= 1.
 * A plan carries the sq and sk it was made for; an attention call whose sizes
 * differ ignores it (built-in order).  A plan made from other positions of
 * the same sizes is still a valid order (same results, other speed).
 * Errors: NULL pointer (MMSP_ERR_NULL), sq or sk < 1 (MMSP_ERR_SHAPE),
 * plan_bytes too small (MMSP_ERR_WORKSPACE; also from the attention calls
 * given a non-NULL plan).  mmsp_attn_packed_plan_bytes returns 0 for sizes
 * below 1.  Cost: one small launch for sq, sk <= 8192 (two per chunk above);
 * tile lists longer than 32768 entries are left in index order.
 *
 * mmsp_attn_packed_plans: the plans of n_chunks chunks in one launch, for
 * chunks whose key positions lie back to back in k_pos (chunk c at
 * k_pos + c * sk, as the slices of one balance permutation do); plan c is
 * written at byte offset c * mmsp_attn_packed_plan_bytes(sq, sk) of `plans`,
 * plans_bytes >= n_chunks times that (else MMSP_ERR_WORKSPACE).
 * 1 <= n_chunks <= 1024 and n_chunks * sk < 2^31 (else MMSP_ERR_SHAPE).
 * mmsp_attn_packed_plan is the case n_chunks = 1.
 */
size_t mmsp_attn_packed_plan_bytes(int32_t sq, int32_t sk);
int mmsp_attn_packed_plan(const int32_t* q_pos, const int32_t* q_start, const int32_t* k_pos,
                          int32_t sq, int32_t sk, void* plan, size_t plan_bytes,
                          hipStream_t stream);
int mmsp_attn_packed_plans(const int32_t* q_pos, const int32_t* q_start, const int32_t* k_pos,
                           int32_t n_chunks, int32_t sq, int32_t sk, void* plans,
                           size_t plans_bytes, hipStream_t stream);

/* ---- a3: log-sum-exp merge of two chunk results ---------------------------
 * The page's ring loop ("Implementation ...") adds each step's output into an
 * accumulator; the exact form of that accumulation over disjoint key sets is
 *   L = ln(e^La + e^Lb),  O = e^(La-L) O_a + e^(Lb-L) O_b,
 * with (0, -inf) as identity and two empty rows giving (0, -inf).
 *
 * o_acc fp32 [sq][hq][d], lse_acc fp32 [hq][sq]: updated in place.
 * o_part, lse_part: the other operand (same layouts); both NULL means "no
 *   operand": only o_final_bf16 is produced from (o_acc, lse_acc).
 * o_final_bf16 (nullable): bf16 [sq][hq][d] copy of the merged o
 *   (round-to-nearest-even).  d in {64, 128}.
 */
int mmsp_lse_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                   int32_t sq, int32_t hq, int32_t d, void* o_final_bf16, hipStream_t stream);

/* ---- a5: backward preprocess ----------------------------------------------
 * delta[h][i] = sum_c dout[i][h][c] * o[i][h][c] (fp32 accumulation) from the
 * saved final output; o, dout bf16 [sq][hq][d]; delta fp32 [hq][sq].
 * dq_zero (nullable) fp32 [sq][hq][d] is set to 0 in the same pass, ready to
 * be the dq_acc of the following mmsp_attn_bwd_chunk calls.
 */
int mmsp_attn_bwd_preprocess(const void* o, const void* dout, int32_t sq, int32_t hq, int32_t d,
                             float* delta, float* dq_zero, hipStream_t stream);

/* ---- a6: backward of one chunk from the saved final LSE --------------------
 * Training without gradient checkpointing ("LongVILA - ... (Jason's Study)",
 * section "What it is"): P = exp(scale*q.k - LSE_final) on visible pairs,
 *   dV = P^T dO,  dS = P o (dO V^T - delta),  dQ += scale dS K,
 *   dK = scale dS^T Q,
 * with dK, dV of a KV head summed over its hq/hkv query heads.
 *
 * q, dout bf16 [sq][hq][d]; k, v bf16 [sk][hkv][d]; lse, delta fp32 [hq][sq]
 * (lse = final merged LSE over all chunks; rows with lse = -inf contribute
 * nothing); q_pos/k_pos as in mmsp_attn_fwd_chunk.
 * dq_acc fp32 [sq][hq][d]: this chunk's dQ is ADDED (zero it before the first
 *   chunk).  Each element is read, summed and written once per call by one
 *   thread (no atomics), so results are deterministic run to run.
 * dk, dv fp32 [sk][hkv][d]: overwritten, or added to with MMSP_ACCUMULATE.
 * Two kernels are enqueued on the stream (dK/dV, then dQ); the call must not
 *   overlap another call that writes the same dq_acc, dk or dv.
 * flags MMSP_BWD_NO_DQ / MMSP_BWD_NO_DKDV enqueue only the other kernel
 *   (dq_acc, or dk and dv, may then be NULL; both flags: MMSP_ERR_UNSUPPORTED).
 *   The two halves read the same inputs and write disjoint outputs, so they
 *   may run on two streams at once.
 */
enum { MMSP_BWD_NO_DQ = 4u, MMSP_BWD_NO_DKDV = 8u };
int mmsp_attn_bwd_chunk(const void* q, const void* k, const void* v, const void* dout,
                        const float* lse, const float* delta, const int32_t* q_pos,
                        const int32_t* k_pos, int32_t sq, int32_t sk, int32_t hq, int32_t hkv,
                        int32_t d, float scale, uint32_t flags, float* dq_acc, float* dk,
                        float* dv, hipStream_t stream);

/* ---- a6 with packed samples -------------------------------------------------
 * As mmsp_attn_bwd_chunk with the packed-sample visibility of
 * mmsp_attn_fwd_chunk_packed (q_start as there; flags must include
 * MMSP_CAUSAL); lse is the final LSE of the packed forward.  plan and
 * plan_bytes as in mmsp_attn_fwd_chunk_packed.
 */
int mmsp_attn_bwd_chunk_packed(const void* q, const void* k, const void* v, const void* dout,
                               const float* lse, const float* delta, const int32_t* q_pos,
                               const int32_t* q_start, const int32_t* k_pos, const void* plan,
                               size_t plan_bytes, int32_t sq, int32_t sk, int32_t hq,
                               int32_t hkv, int32_t d, float scale, uint32_t flags,
                               float* dq_acc, float* dk, float* dv, hipStream_t stream);

/* ---- a4: one rank's ring loop over resident chunks -----------------------
 * "LongVILA Guide ...", section "Implementation: PyTorch Distributed
 * Pipeline and Token Routing": at ring step t a rank computes attention of
 * its local queries against the chunk it holds, which came from rank
 * (rank - t) mod P; section "Multi-Modal Sequence Parallelism (MM-SP)
 * Mechanics", item 3: one kernel per step.  With all n_chunks chunks resident,
 * these calls visit chunk (rank - t) mod n_chunks at step t and make the same
 * launches, in the same order, as calling the chunk entry points one by one.
 *
 * k_chunks, v_chunks (bf16 [sk][hkv][d]), k_pos_chunks (int32 [sk]), and for
 * the backward dk_chunks, dv_chunks (fp32 [sk][hkv][d]): HOST arrays of
 * n_chunks DEVICE pointers, read during the call only.  Every chunk has sk
 * keys.  q, q_pos, q_start, scale and the shapes are as in
 * mmsp_attn_fwd_chunk(_packed); q_start (nullable) selects packed samples
 * and needs MMSP_CAUSAL (these loops use the built-in tile order: no tile
 * plan).  0 <= rank < n_chunks.
 *
 * mmsp_ring_forward: the first step writes (o fp32 [sq][hq][d], lse fp32
 *   [hq][sq]), later steps merge into them (MMSP_ACCUMULATE); then, if
 *   o_final_bf16 is not NULL, the bf16 output [sq][hq][d] is written as
 *   mmsp_lse_merge does.  flags: MMSP_CAUSAL or 0.
 * mmsp_ring_backward: delta (fp32 [hq][sq]) from o_bf16 and dout with dq
 *   (fp32 [sq][hq][d]) zeroed, as mmsp_attn_bwd_preprocess; then one backward
 *   per chunk in ring order: dq accumulates every chunk's contribution and
 *   dk_chunks[c], dv_chunks[c] are overwritten (added to with
 *   MMSP_ACCUMULATE).  lse is the final LSE of the forward.  flags:
 *   MMSP_CAUSAL and/or MMSP_ACCUMULATE.
 *
 * Errors: every argument of every chunk is checked before the first launch
 * (NULL array or entry: MMSP_ERR_NULL; n_chunks <= 0 or rank out of range:
 * MMSP_ERR_SHAPE; other codes as the chunk entry points).  MMSP_ERR_HIP from
 * a launch part-way returns at once and leaves the earlier launches
 * enqueued.
 */
int mmsp_ring_forward(const void* q, const void* const* k_chunks, const void* const* v_chunks,
                      const int32_t* q_pos, const int32_t* const* k_pos_chunks,
                      const int32_t* q_start, int32_t n_chunks, int32_t rank, int32_t sq,
                      int32_t sk, int32_t hq, int32_t hkv, int32_t d, float scale,
                      uint32_t flags, float* o, float* lse, void* o_final_bf16, hipStream_t stream);
int mmsp_ring_backward(const void* q, const void* const* k_chunks, const void* const* v_chunks,
                       const void* dout, const void* o_bf16, const float* lse,
                       const int32_t* q_pos, const int32_t* const* k_pos_chunks,
                       const int32_t* q_start, int32_t n_chunks, int32_t rank, int32_t sq,
                       int32_t sk, int32_t hq, int32_t hkv, int32_t d, float scale,
                       uint32_t flags, float* delta, float* dq, float* const* dk_chunks,
                       float* const* dv_chunks, hipStream_t stream);

/* ---- rotary position embedding at global positions ------------------------
 * "LongVILA Guide ...", section "Three-Stage Long-Context Alignment
 * Curriculum", stage 2: the rotary base theta is raised to 10,000,000 for the
 * long-context stages.  Half-split pairs (x[i], x[i+d/2]) of the token at
 * position pos[t] turn by the angle pos[t] * theta^(-2i/d); with inverse = 1
 * by minus that angle (the transpose: it maps gradients with respect to the
 * rotated queries/keys to gradients with respect to the unrotated ones).
 *
 * x, y   [s][h][d] of `dtype` (MMSP_DTYPE_BF16 or MMSP_DTYPE_F32); y may equal
 *        x (in place).
 * pos    int32 [s]: the tokens' global positions (e.g. a shard's q_pos).
 * Angles are formed in fp64 from the integer positions; bf16 results are
 * rounded fp64 -> fp32 -> bf16 (nearest even), fp32 results fp64 -> fp32.
 * d in {64, 128} and inverse in {0, 1} (else MMSP_ERR_UNSUPPORTED); s, h >= 1,
 * s*h*d < 2^31, theta > 1 and finite (else MMSP_ERR_SHAPE).  Memory-bound,
 * one pass.
 * Rotate a rank's Q and its own K chunk once per layer, before the ring (the
 * chunk then travels rotated), and apply the inverse to dQ and to each dK
 * after the backward.
 */
enum { MMSP_DTYPE_BF16 = 0, MMSP_DTYPE_F32 = 1 };

int mmsp_rope(const void* x, void* y, int32_t dtype, const int32_t* pos, int32_t s, int32_t h,
              int32_t d, double theta, int32_t inverse, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MMSP_H */
