/*
 * attnring.h - C ABI of the blockwise causal GQA ring-attention library (gfx950).
 *
 * The operation: context-parallel prefill splits a prompt along the sequence,
 * and Ring Attention has each device run attention with its partial query
 * against partial key/value blocks while the key/value blocks travel to its
 * ring neighbours (Moreh, "Optimizing Long-Context Prefill on Multiple
 * Older-Generation GPU Nodes", section "Introduction to Context Parallelism",
 * the context-parallelism paragraph and the Ring Attention bullet).  The
 * partial results must add up to ordinary causal attention over the whole
 * sequence.  This library provides the device-side pieces of that:
 *
 *   attn_ring_step      - attention of the local query block against ONE
 *                         key/value block, producing a partial (O, LSE);
 *   attn_ring_step_merge - the same step folded straight into a running
 *                         (O, LSE) in place, with no partial buffers;
 *   attn_ring_merge     - folds a partial (O, LSE) into a running one;
 *   attn_prefill_causal - full causal attention in one call (the result the
 *                         ring must reproduce, and the N = 1 case).
 *
 * Definition (per packed sequence b, query row p, query head h):
 *   g        = h / (Hq / Hkv)                 (query heads in consecutive groups
 *                                              share one key/value head)
 *   s[p,k]   = scale * dot(q[p,h,:], k[k,g,:])
 *   visible  = keys k of sequence b with kpos(k) <= qpos(p) when causal, all
 *              keys of sequence b otherwise; kpos/qpos are global positions
 *   LSE[h,p] = ln sum_{visible} exp(s[p,k])   (natural log; -inf if none)
 *   O[p,h,:] = sum_{visible} exp(s[p,k] - LSE[h,p]) * v[k,g,:]   (0 if none)
 *
 * Layouts (all row-major, contiguous, device memory):
 *   q         [total_q, Hq,  head_dim]   bf16 or fp32 (attn_dtype)
 *   k, v      [total_k, Hkv, head_dim]   same dtype as q
 *   o         [total_q, Hq,  head_dim]   fp32
 *   lse       [Hq, total_q]              fp32
 * Several sequences may be packed along the token axis: rows
 * [cu_q[b], cu_q[b+1]) of q and [cu_k[b], cu_k[b+1]) of k/v belong to
 * sequence b; q_pos0[b] / k_pos0[b] give the global position of each
 * sequence's first row in this block (a rank's chunk starts mid-sequence).
 *
 * Ownership and execution: the caller allocates and owns every buffer; the
 * library allocates, frees and synchronises nothing.  Host arrays in
 * attn_problem are read during the call only.  Work is enqueued on `stream`
 * (NULL = the default stream) and runs asynchronously; device faults surface
 * at the caller's next synchronisation.
 *
 * Errors: every argument is validated on the host before anything is
 * enqueued.  On a non-OK status nothing was enqueued (except ATTN_EHIP,
 * returned when the launch itself failed), and attn_last_error() gives a
 * message.  The library keeps no other state and is thread-safe.
 */
#ifndef ATTNRING_H
#define ATTNRING_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 3
#define ATTN_MAX_SEQS 64 /* packed sequences per call (their tables travel in kernel arguments) */

typedef enum { ATTN_DTYPE_BF16 = 0, ATTN_DTYPE_FP32 = 1 } attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,       /* an argument is invalid; nothing enqueued */
  ATTN_EUNSUPPORTED = 2, /* valid but not implemented (head_dim != 64, or with bf16 one
                            sequence's k or v spanning 2 GiB or more); nothing enqueued */
  ATTN_EHIP = 3          /* the HIP launch failed */
} attn_status;

typedef struct {
  int32_t num_seqs;       /* B, 1 <= B <= ATTN_MAX_SEQS */
  const int32_t* cu_q;    /* HOST [B+1] prefix row offsets into q; NULL means B == 1, [0, total_q] */
  const int32_t* cu_k;    /* HOST [B+1] prefix row offsets into k/v; NULL means B == 1, [0, total_k] */
  const int32_t* q_pos0;  /* HOST [B] global position of each sequence's first q row; NULL = all 0 */
  const int32_t* k_pos0;  /* HOST [B] global position of each sequence's first k row; NULL = all 0 */
  int32_t total_q;        /* rows of q (>= 0) */
  int32_t total_k;        /* rows of k and v (>= 0) */
  int32_t num_q_heads;    /* Hq >= 1 */
  int32_t num_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;       /* 64 */
  float scale;            /* > 0 and finite; 0 selects 1/sqrt(head_dim) */
  int32_t causal;         /* 1: mask keys whose position exceeds the query's; 0: no mask */
  /* Optional explicit key ranges, instead of cu_k (which must then be NULL): sequence b's
   * keys are rows k_row0[b] .. k_row0[b] + k_len[b] - 1 of k/v.  HOST [B] arrays, both or
   * neither; ranges may overlap or come in any order (two query segments can attend to
   * the same keys, as in load-balanced zigzag rings).  Not accepted by attn_prefill_causal. */
  const int32_t* k_row0;
  const int32_t* k_len;
} attn_problem;

/*
 * One ring step: attention of the local query rows against one key/value
 * block.  Writes the partial result of every local row to o_part / lse_part
 * (rows with no visible key get O = 0, LSE = -inf, the merge identity).
 *
 * Fully masked step: when no sequence has a visible key in this block (the
 * block lies wholly in the future of the local rows), nothing needs to run.
 * If `launched` is non-NULL the call then enqueues nothing, sets *launched =
 * 0, and the caller must skip the merge for this step; otherwise the identity
 * is written so a following merge stays correct.  *launched = 1 whenever the
 * outputs were written.
 *
 * q, k, v, o_part: 16-byte aligned; lse_part: 4-byte aligned.  o_part and
 * lse_part must not overlap the inputs.
 */
attn_status attn_ring_step(const attn_problem* problem, attn_dtype dtype,
                           const void* q, const void* k, const void* v,
                           float* o_part, float* lse_part,
                           int32_t* launched, hipStream_t stream);

/*
 * One ring step fused with its merge: attention of the local query rows
 * against one key/value block, folded by log-sum-exp straight into the
 * running state (o_acc, lse_acc) in place.  The result equals attn_ring_step
 * into separate buffers followed by attn_ring_merge (up to rounding), without
 * the partial buffers or the second pass over them.
 *
 * o_acc [total_q, Hq, head_dim] and lse_acc [Hq, total_q] are fp32, read and
 * written; they must hold a valid running state (finite O; a row with no keys
 * yet is (0, -inf)).  Rows that see no key in this block are left untouched;
 * a block with no visible key at all enqueues nothing.  *launched (if
 * non-NULL) is 1 when a kernel was enqueued, else 0.  Alignment and overlap
 * rules are those of attn_ring_step.
 */
attn_status attn_ring_step_merge(const attn_problem* problem, attn_dtype dtype,
                                 const void* q, const void* k, const void* v,
                                 float* o_acc, float* lse_acc,
                                 int32_t* launched, hipStream_t stream);

/*
 * Merge of two partial results over disjoint key sets (the step that lets the
 * ring's partial results add up to full attention), in place on the running
 * state:  M = max(La, Lb);  L = M + ln(e^(La-M) + e^(Lb-M));
 *         O = e^(La-L) * Oa + e^(Lb-L) * Ob.
 * (0, -inf) is the identity; two empty partials stay (0, -inf).
 * o_acc/o_part are [total_q, Hq, head_dim] fp32, lse_acc/lse_part are
 * [Hq, total_q] fp32.  o_part must not overlap o_acc, nor lse_part lse_acc.
 * o buffers 16-byte aligned.
 */
attn_status attn_ring_merge(int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                            float* o_acc, float* lse_acc,
                            const float* o_part, const float* lse_part,
                            hipStream_t stream);

/*
 * Full causal prefill in one call: every packed sequence attends causally to
 * itself.  Requires causal == 1, cu_k equal to cu_q (or both NULL),
 * total_k == total_q, and q_pos0 / k_pos0 NULL or equal to each other.
 * Writes final O and LSE for every row.
 */
attn_status attn_prefill_causal(const attn_problem* problem, attn_dtype dtype,
                                const void* q, const void* k, const void* v,
                                float* o, float* lse, hipStream_t stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* attn_last_error(void);

/* ATTN_ABI_VERSION of the built library. */
int32_t attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRING_H */
