/*
 * bdlm_attn.h -- C ABI of the BDLM masked-attention library for AMD MI355X (gfx950).
 *
 * The operation (from "Block Parallelism For Efficient Distributed Long-Context
 * Diffusion Language Model Training", arXiv 2609.19242; abstract and the
 * evolve.pub review's Summary, Strengths and FAQ):
 *
 *   A block diffusion LM trains on the concatenation [x0 ; xt] of L clean and L
 *   corrupted tokens split into blocks of B tokens.  Across blocks the model is
 *   autoregressive; inside a block the corrupted tokens are denoised in parallel.
 *   Clean K/V are shared by every later block, corrupted K/V belong to their own
 *   block.  Per (batch, q-head h, kv-head g = h / (Hq/Hkv)):
 *     - a clean query of block b sees the clean keys of blocks <= b;
 *     - a corrupted query of block b sees the clean keys of blocks < b and the
 *       corrupted keys of block b;
 *     - S = scale * <q, k>, LSE = log sum_{visible} exp(S) (natural log),
 *       P = exp(S - LSE) on visible pairs, O = P V.
 *   Backward (LSE gets no gradient): D = rowsum(dO * O), dP = dO V^T,
 *   dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO, dK/dV of a
 *   kv head summed over the q heads that read it.
 *
 *   Because the objective separates over target blocks (block parallelism, BP)
 *   a rank can compute whole corrupted blocks against the clean prefix, and the
 *   clean sequence can be sharded (context-sharded BP, CSBP): a block's output
 *   is then assembled from partials over disjoint clean-key chunks, merged by
 *   their log-sum-exp; the result equals the length-2L computation up to
 *   floating-point reduction order (review: Strengths, Prop. 1 / App. A).
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers owned by the caller, 16-byte aligned,
 *     dense row-major.  Q/K/V/O/dO/dQ/dK/dV use [batch, tokens, heads, head_dim];
 *     LSE uses [batch, Hq, tokens] fp32.
 *   - Element type is desc->dtype (BDLM_F32 or BDLM_BF16) unless stated fp32.
 *   - Calls are asynchronous on `stream` (0 = the null stream).  Every argument and
 *     every launch size is validated before anything is enqueued; on such an error
 *     the call returns a non-zero bdlm_status, enqueues nothing and leaves all
 *     outputs untouched.  BDLM_ERR_HIP (the runtime refusing a launch) is the one
 *     exception: a call that launches several kernels (bdlm_attn_bwd) may then
 *     have enqueued the launches before the refused one.
 *   - No call allocates device memory.  Scratch memory is the caller's `ws`
 *     buffer of at least bdlm_attn_workspace_bytes() bytes, which must stay
 *     alive, and not be shared with a concurrent call, until the stream reaches
 *     the end of the call.
 *   - Device faults surface at the caller's next synchronisation.  Calls on
 *     distinct streams with distinct workspaces are thread-safe.
 *   - Constraints: L % B == 0, B % 16 == 0, Hq % Hkv == 0, head_dim in {64, 128},
 *     batch, L, heads >= 1.
 */
#ifndef BDLM_ATTN_H
#define BDLM_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BDLM_OK = 0,
  BDLM_ERR_INVALID_ARG = 1, /* a shape, pointer, window or id list is invalid */
  BDLM_ERR_UNSUPPORTED = 2, /* valid but not built (head_dim, too many blocks/parts) */
  BDLM_ERR_WORKSPACE = 3,   /* ws is NULL or smaller than bdlm_attn_workspace_bytes() */
  BDLM_ERR_HIP = 4          /* the HIP runtime refused a launch */
} bdlm_status;

typedef enum { BDLM_F32 = 0, BDLM_BF16 = 1 } bdlm_dtype;

#define BDLM_MAX_LOCAL_BLOCKS 256
#define BDLM_MAX_MERGE_PARTS 64

/* Problem descriptor (plain data, read during the call only). */
typedef struct {
  int32_t batch;          /* >= 1                                                 */
  int32_t seqlen;         /* L: clean tokens; in full mode also corrupted tokens  */
  int32_t block;          /* B                                                    */
  int32_t num_q_heads;    /* Hq                                                   */
  int32_t num_kv_heads;   /* Hkv, divides Hq (GQA: q head h reads kv head h/(Hq/Hkv)) */
  int32_t head_dim;       /* 64 or 128                                            */
  int32_t dtype;          /* bdlm_dtype of Q/K/V/O/dO/dQ/dK/dV                     */
  float softmax_scale;    /* s in S = s <q, k>; must be finite and > 0            */
  /* CSBP share mode when num_local_blocks > 0: the queries are whole corrupted
     blocks of one rank, attending to one clean-key window and (optionally) to
     their own corrupted block. */
  int32_t num_local_blocks;   /* 0 = full mode; else 1..BDLM_MAX_LOCAL_BLOCKS      */
  const int32_t* block_ids;   /* HOST array [num_local_blocks]: global block index of
                                 each local block, strictly increasing, < L/B       */
  int32_t kv_begin, kv_end;   /* clean-key window [kv_begin, kv_end) of this call,
                                 0 <= kv_begin <= kv_end <= L                       */
  int32_t own_block;          /* 1 = also attend each block's own corrupted K/V     */
  /* Share mode only: 1 = the local blocks are CLEAN query blocks (the rank's
     shard of the clean stream in context-parallel form): block i then sees the
     clean keys of its own and all earlier blocks, [0, (block_ids[i]+1)*B), cut
     to the window; own_block must be 0.  0 = corrupted blocks (strict clean
     prefix).  Must be 0 in full mode.                                           */
  int32_t clean_queries;
  /* Share mode, forward only (the backward ignores it): 1 = merge this call's
     partial into the (O, LSE) that ox / lse_x already hold from earlier calls
     of the same stream of chunks, in place (the running merge fused into the
     kernel's epilogue); 0 = overwrite them with this call's partial.  Must be 0
     in full mode. */
  int32_t accumulate;
  /* Share mode only: 1 = kc, vc (and in the backward dkc, dvc) hold just this
     call's window, rows [kv_begin, kv_end) of the clean sequence, as
     [batch, kv_end - kv_begin, Hkv, d]: a chunk-sized staging buffer, the way a
     rank receives a shard of the clean K/V from an all-gather and hands the
     chunk's clean dK/dV to a reduce-scatter (pages: review FAQ "What is CSBP?",
     the clean sequence sharded and only clean K/V and their gradients
     exchanged).  0 = they hold the whole clean sequence [batch, L, Hkv, d].
     Must be 0 in full mode. */
  int32_t kv_staged;
} bdlm_attn_desc;

/* Bytes of scratch memory a call needs (0 is possible).  for_bwd selects
   bdlm_attn_bwd (1) or bdlm_attn_fwd (0).  Returns 0 for an invalid desc. */
size_t bdlm_attn_workspace_bytes(const bdlm_attn_desc* desc, int for_bwd);

/* Validate `desc` only (no device work).  Returns a bdlm_status. */
int bdlm_attn_check_desc(const bdlm_attn_desc* desc);

/*
 * Forward.
 * Full mode (num_local_blocks == 0):
 *   qc, qx [batch, L, Hq, d]; kc, vc, kx, vx [batch, L, Hkv, d] (c = clean x0,
 *   x = corrupted xt).  Writes oc, ox [batch, L, Hq, d] (dtype) and
 *   lse_c, lse_x [batch, Hq, L] fp32.
 * Share mode (num_local_blocks = n > 0):
 *   qc, oc, lse_c must be NULL.  qx [batch, n*B, Hq, d] and kx, vx
 *   [batch, n*B, Hkv, d] hold the local corrupted blocks in block_ids order;
 *   kc, vc [batch, L, Hkv, d] are the whole clean sequence, of which only rows
 *   [kv_begin, kv_end) are read.  Local block i sees clean keys
 *   [kv_begin, min(kv_end, block_ids[i]*B)) and, if own_block, its own rows
 *   [i*B, (i+1)*B) of kx/vx (kx, vx may be NULL when own_block is 0).  With
 *   clean_queries = 1, qx holds clean query blocks and block i sees clean keys
 *   [kv_begin, min(kv_end, (block_ids[i]+1)*B)): the clean stream's rule that a
 *   clean block attends to itself and every earlier clean block (pages: Block
 *   Parallelism ..., Sec. 4 and Fig. 3, the clean sequence sharded across the
 *   ranks in context-parallel form).  Writes the PARTIAL result over exactly those keys
 *   to ox (fp32, [batch, n*B, Hq, d]) and lse_x (fp32, [batch, Hq, n*B]); rows
 *   that see no key get O = 0 and LSE = -inf.  With accumulate = 1 the partial
 *   is instead merged into the (O, LSE) that ox / lse_x hold: LSE becomes
 *   logsumexp(LSE_held, LSE_part) and O the exp(LSE_j - LSE)-weighted sum of the
 *   two (pages: the clean prefix streamed in chunks and the per-block results
 *   combined, Sec. 4 / Fig. 3 as the review describes CSBP); rows that see no
 *   key in this call are left as they are.  The caller starts a stream of
 *   chunks with accumulate = 0 and must not run two accumulating calls on the
 *   same ox / lse_x at once.
 */
int bdlm_attn_fwd(const bdlm_attn_desc* desc,
                  const void* qc, const void* kc, const void* vc,
                  const void* qx, const void* kx, const void* vx,
                  void* oc, void* ox, float* lse_c, float* lse_x,
                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward of bdlm_attn_fwd.  The gradients are those of the length-2L masked
 * attention over [x0 ; xt]; in share mode they are the block-separated terms
 * whose sum over the streamed clean chunks (and the own block) equals it up to
 * floating-point reduction order: the objective separates over target blocks,
 * so a corrupted block's gradients can be formed on one rank against the clean
 * prefix, and the clean K/V gradients of a chunk are what CSBP returns to the
 * chunk's owner (pages: review Strengths, Prop. 1 / App. A, exactness of BP;
 * FAQ "What is CSBP?", only clean K/V and their gradients are exchanged).
 * Stored-LSE recompute (P is rebuilt from Q, K and LSE):
 * D = rowsum(dO * O) (with LSE * log2(e), kept in the workspace: fp32
 * [batch, Hq, rows] each, per query stream), then dK/dV key-major and dQ
 * query-major (no atomics).
 * Full mode: inputs as the forward plus its outputs oc, ox, lse_c, lse_x and the
 *   upstream gradients doc, dox [batch, L, Hq, d].  Overwrites dqc, dqx
 *   [batch, L, Hq, d] and dkc, dvc, dkx, dvx [batch, L, Hkv, d] (all dtype).
 * Share mode: qc, oc, lse_c, doc, dqc must be NULL.  ox is the FINAL (merged)
 *   output [batch, n*B, Hq, d] in dtype and lse_x the final LSE.  For the keys of
 *   this call's window:
 *     - ADDS the dQ contribution into dqx, which is fp32 [batch, n*B, Hq, d]
 *       (the caller zeroes it once before the first chunk);
 *     - overwrites rows [kv_begin, kv_end) of dkc, dvc ([batch, L, Hkv, d], dtype;
 *       rows no local block sees get 0; other rows are untouched);
 *     - if own_block, overwrites dkx, dvx [batch, n*B, Hkv, d] (dtype); else
 *       dkx, dvx (and kx, vx) may be NULL and are not touched.
 *   clean_queries selects the clean-query rule as in the forward.
 */
int bdlm_attn_bwd(const bdlm_attn_desc* desc,
                  const void* qc, const void* kc, const void* vc,
                  const void* qx, const void* kx, const void* vx,
                  const void* oc, const void* ox, const float* lse_c, const float* lse_x,
                  const void* doc, const void* dox,
                  void* dqc, void* dkc, void* dvc, void* dqx, void* dkx, void* dvx,
                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * bdlm_attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving or training loops,
 * harnesses that forbid allocation calls).  Same arguments, semantics and
 * results as bdlm_attn_bwd (the same kernels run), minus ws / ws_bytes: the
 * workspace is a fixed array of bdlm_attn_noalloc_scratch_bytes() bytes (64 MiB)
 * that is part of the library's device image, one copy per GPU, held until the
 * process ends.  The call uses the copy of the CURRENT device (the stream must
 * belong to it) and allocates nothing.
 *   - A problem whose workspace (bdlm_attn_workspace_bytes(desc, 1)) exceeds the
 *     array returns BDLM_ERR_UNSUPPORTED before anything is enqueued.  The
 *     limit admits batch * Hq * rows <= 4M (query rows of both streams counted
 *     once: e.g. 32 q heads at L = 131072).
 *   - Nothing in the array must start at zero: every call writes the parts it
 *     reads before reading them.
 *   - Every call on one GPU shares that GPU's array: calls that may overlap in
 *     time (different streams, or the same stream from different threads
 *     without ordering) race on it and must not be issued.
 * Returns BDLM_ERR_HIP if the device or the array's address cannot be found.
 */
int bdlm_attn_bwd_noalloc(const bdlm_attn_desc* desc,
                          const void* qc, const void* kc, const void* vc,
                          const void* qx, const void* kx, const void* vx,
                          const void* oc, const void* ox, const float* lse_c, const float* lse_x,
                          const void* doc, const void* dox,
                          void* dqc, void* dkc, void* dvc, void* dqx, void* dkx, void* dvx,
                          hipStream_t stream);

/* Size in bytes of the per-GPU workspace array of bdlm_attn_bwd_noalloc. */
size_t bdlm_attn_noalloc_scratch_bytes(void);

/*
 * Merge attention partials over disjoint key sets: the (O, LSE) combination by
 * which a corrupted block's attention over the clean prefix, streamed in chunks
 * under CSBP, is assembled from one partial per chunk; exact up to
 * floating-point reduction order (pages: review FAQ "What is CSBP?", the clean
 * sequence sharded and only clean K/V exchanged; Strengths, Prop. 1 / App. A):
 *   LSE = log sum_j exp(LSE_j),  O = sum_j exp(LSE_j - LSE) O_j.
 * o_parts, lse_parts: HOST arrays of num_parts (1..BDLM_MAX_MERGE_PARTS) DEVICE
 * pointers; O_j fp32 [batch, tokens, heads, head_dim], LSE_j fp32
 * [batch, heads, tokens].  Writes o_out in out_dtype and lse_out (fp32).  A
 * partial with LSE = -inf has weight 0; a row whose partials are all -inf gets
 * O = 0, LSE = -inf.  o_out / lse_out may alias o_parts[0] / lse_parts[0] (fp32
 * out_dtype) for an in-place running merge; no other aliasing is allowed.
 */
int bdlm_attn_merge_partials(int32_t num_parts, int32_t batch, int64_t tokens,
                             int32_t heads, int32_t head_dim,
                             const float* const* o_parts, const float* const* lse_parts,
                             void* o_out, int32_t out_dtype, float* lse_out,
                             hipStream_t stream);

/*
 * Diagnostics: walk a kernel's work decomposition on the host exactly as the
 * kernel traverses it -- for_bwd = 0: forward, 1: backward dK/dV (key-major),
 * 2: backward dQ (query-major, the forward's decomposition) -- for batch 0 and
 * q-head 0, adding 1 to cover[row * keys + key] (saturating at 255) for every
 * (query row, key) pair the kernels treat as visible.  Rows are the query rows
 * of stream 0 followed by stream 1 (full mode: 2L rows; share mode: 0 + n*B);
 * keys are key array 0 followed by array 1 (full: 2L; share: L + n*B).  cover
 * may be NULL; otherwise cover_len must hold rows * keys bytes.  stats (may be
 * NULL) receives 5 values: {workgroups launched, tile visits, tile visits
 * needing the element mask, pairs marked, consistency errors}.  No device work.
 */
int bdlm_attn_schedule_walk(const bdlm_attn_desc* desc, int for_bwd, uint8_t* cover,
                            int64_t cover_len, int64_t* stats);

/* Human-readable name of a bdlm_status value (static string). */
const char* bdlm_status_str(int status);

/* Library ABI version (major * 100 + minor). */
int bdlm_attn_version(void);

/*
 * Kernel timing (diagnostics).  While enabled, every kernel the library
 * launches is bracketed by HIP events on its stream.  bdlm_attn_profile_begin
 * creates a pool of `max_launches` event pairs (the only calls that create HIP
 * objects); bdlm_attn_profile_end synchronises those events, writes up to
 * `max_entries` per-kernel totals and destroys the pool.  Not thread-safe.
 */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} bdlm_kernel_time;

int bdlm_attn_profile_begin(int32_t max_launches);
int bdlm_attn_profile_end(bdlm_kernel_time* out, int32_t max_entries, int32_t* num_entries);

/*
 * Calibration (diagnostics; not part of the attention path): the bf16 MFMA
 * rate the chip sustains under a given operand and instruction mix.  The
 * published dense peak assumes the 2.4 GHz peak clock; under load the chip
 * holds its power limit by lowering the clock, and how far depends on the
 * operand bits that toggle.  Launches `workgroups` workgroups of 8 waves (two
 * per SIMD, one workgroup per CU) on `stream`; every wave runs `iters` (even,
 * >= 2) steps of 4 v_mfma_f32_32x32x16_bf16 (32768 flop each) on four
 * independent accumulators, plus per mode:
 *   0  constant operands;
 *   1  random operands (bf16 uniform in [-0.5, 0.5), 8 register sets in turn);
 *   2  mode 1 plus one 16-byte LDS read per lane per MFMA (1 KB per wave and
 *      MFMA, the attention kernels' LDS operand traffic), read 4 MFMAs ahead;
 *   3  mode 1 plus 4 FMAs per MFMA.
 * cycles: device int64 [workgroups * 8 * 2], per wave {shader-clock cycles,
 * 100 MHz real-time ticks} over its MFMA loop (clock = cycles / ticks * 0.1 GHz).
 * sink: device float [workgroups * 512], written so no work is removed.  The
 * caller times the launch (events on `stream`): rate = workgroups * 8 * iters
 * * 4 * 32768 flop / time.  Returns BDLM_ERR_INVALID_ARG before any device work
 * for a bad mode, size or null pointer, BDLM_ERR_HIP if the launch fails.
 */
int bdlm_calib_mfma(int32_t mode, int32_t workgroups, int32_t iters, int64_t* cycles, float* sink,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BDLM_ATTN_H */
