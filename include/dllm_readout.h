/*
 * dllm_readout.h -- C ABI of the masked-token readout of a masked diffusion
 * LLM on AMD Instinct MI355X (gfx950).
 *
 * One call of dllm_masked_readout_step is one denoising readout:
 *   1. gather the final hidden states of positions that still hold the mask
 *      token ("mask-only logits": Mosaic, Unlocking Long-Context Inference for
 *      Diffusion LLMs via Global Memory Planning and Dynamic Peak Taming,
 *      TL;DR and Abstract);
 *   2. project them through the LM head W_lm [V, d];
 *   3. reduce every row over the vocabulary in vocab-chunked streaming form
 *      (running max, argmax and sum of exponentials), so the L x V logits
 *      tensor -- the memory peak at high mask ratio in Mosaic Fig. 3 -- never
 *      exists; each row yields its argmax token, its confidence (largest
 *      softmax probability) and its log-sum-exp;
 *   4. commit the k most confident candidates (confidence-driven unmasking:
 *      Accelerating Masked Diffusion Large Language Models: A Survey of
 *      Efficient Inference Techniques, Main Findings), writing their tokens
 *      into the sequence and clearing their mask flags, as the sequence goes
 *      from fully masked to unmasked over T steps (Sparse-dLLM: Accelerating
 *      Diffusion LLMs with Dynamic Cache Eviction, Method "Inference
 *      background").
 *
 * Ties: a row's argmax is the lowest vocabulary index among equal maxima;
 * among equal confidences the lowest position is committed first.
 *
 * Memory: every pointer is a DEVICE pointer unless marked "host".  bf16 data
 * is passed as uint16_t bit patterns.  Arrays are row-major and contiguous.
 * The caller owns and allocates everything (W_lm, hidden, mask, tokens,
 * workspace, outputs); the library never allocates device memory.  The
 * handle is a small host object.
 *
 * Streams: all work of a step is queued on the handle's stream and the call
 * returns without waiting; the caller synchronises before reading results.
 * A step queues kernel launches only (plus the two event records of
 * dllm_masked_readout_set_gemm_events when set): no memset, copy, allocation
 * or host synchronisation, so it may be captured in a HIP graph on the
 * handle's stream; each replay is one step on the captured buffers.
 * A handle is not thread-safe; several handles may share one W_lm.
 *
 * Errors: arguments are checked on the host before anything is queued; on
 * an argument error nothing is written.  DLLM_ERR_HIP reports a failed HIP
 * call or launch; mask and tokens are then unspecified.
 */
#ifndef DLLM_READOUT_H
#define DLLM_READOUT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dllm_readout dllm_readout; /* opaque host-side handle */

typedef enum {
  DLLM_OK = 0,
  DLLM_ERR_INVALID_ARG = 1, /* null pointer, size or range out of bounds */
  DLLM_ERR_UNSUPPORTED = 2, /* shape not divisible as required, pointer misaligned, size over a limit */
  DLLM_ERR_WORKSPACE = 3,   /* workspace null or smaller than dllm_masked_readout_workspace_bytes */
  DLLM_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed (also: no GPU) */
} dllm_status;

/* Largest k_max a handle accepts. */
#define DLLM_K_MAX_LIMIT 4096

/*
 * Optional per-step outputs (host struct of device pointers; each may be
 * NULL).  "Rows" are the candidate positions of the step in ascending
 * position order; there are M of them (M <= the window length).
 *   n_out     [1]      n, the number of committed positions (min(k, M) for
 *                      top-k; the threshold rule of dllm_policy otherwise)
 *   m_out     [1]      M
 *   sel_idx   [k_max]  committed positions in rank order (score
 *                      descending, position ascending); first n valid
 *   sel_tok   [k_max]  their tokens
 *   sel_conf  [k_max]  their confidences (float32)
 *   row_idx   [L_max]  candidate positions, ascending; first M valid
 *   row_tok   [L_max]  argmax token of each candidate row
 *   row_conf  [L_max]  confidence = max softmax probability = exp(max - lse)
 *   row_lse   [L_max]  natural log-sum-exp of the row's logits
 *   row_margin  [L_max]  largest minus second-largest softmax probability
 *                        (0 when the largest logit repeats)
 *   row_entropy [L_max]  -sum_v p_v ln p_v of the row's softmax
 * Asking for row_margin or row_entropy (or ranking by them, dllm_policy)
 * makes the GEMM keep two more running values per row, in the same pass.
 * "Rank order" is by the step's ranking score (dllm_policy); sel_conf always
 * holds confidences.
 */
typedef struct {
  int32_t *n_out;
  int32_t *m_out;
  int32_t *sel_idx;
  int32_t *sel_tok;
  float *sel_conf;
  int32_t *row_idx;
  int32_t *row_tok;
  float *row_conf;
  float *row_lse;
  float *row_margin;
  float *row_entropy;
} dllm_step_out;

/*
 * Ranking score of a candidate row (the unmasking policies the survey
 * groups as confidence- and entropy-driven: Accelerating Masked Diffusion
 * Large Language Models: A Survey of Efficient Inference Techniques, Main
 * Findings).  Larger scores commit first.
 */
typedef enum {
  DLLM_SCORE_CONF = 0,       /* largest softmax probability */
  DLLM_SCORE_MARGIN = 1,     /* largest minus second-largest probability */
  DLLM_SCORE_NEG_ENTROPY = 2 /* minus the softmax entropy (nats) */
} dllm_score;

/*
 * Selection policy of a step.
 *   score          a dllm_score
 *   use_threshold  0: commit the n = min(k, M) best rows (top-k).
 *                  1: adaptive parallel decoding (Dynamic-dLLM, abstract):
 *                  commit every row whose score is >= tau, but at least one
 *                  (the best) and at most k: n = min(max(#{score >= tau}, 1),
 *                  k, M); n = 0 when M = 0 or k = 0.  The comparison is
 *                  made in float32 on the float32 score.
 *   tau            threshold (ignored for top-k); must not be NaN
 */
typedef struct {
  int32_t score;
  int32_t use_threshold;
  float tau;
} dllm_policy;

/*
 * Bytes of device workspace a handle needs for these limits (host-only
 * arithmetic, no HIP call).  Returns 0 if the limits are invalid.
 */
size_t dllm_masked_readout_workspace_bytes(int64_t L_max, int64_t d, int64_t V, int32_t k_max);

/*
 * Create a handle.
 *   out        host: receives the handle (set to NULL on error)
 *   W_lm       [V, d] bf16 LM head, borrowed; must outlive the handle,
 *              16-byte aligned
 *   V, d       vocabulary size (1 <= V < 2^31) and hidden size (d % 8 == 0)
 *   L_max      largest sequence length a step will be called with
 *   k_max      largest unmask count (0 <= k_max <= DLLM_K_MAX_LIMIT)
 *   workspace  device buffer of >= dllm_masked_readout_workspace_bytes(...)
 *              bytes, 256-byte aligned, borrowed; must outlive the handle
 *   stream     hipStream_t to queue work on (NULL = the default stream)
 * Host-only: makes no HIP call and queues no work (the device's compute-unit
 * count is queried by the first step, which returns DLLM_ERR_HIP if there is
 * no usable device).  With the environment variable DLLM_LOG=1 when the
 * handle is created, each of its steps prints the GEMM variant it chose
 * to stderr.
 */
dllm_status dllm_masked_readout_create(dllm_readout **out, const uint16_t *W_lm, int64_t V,
                                       int64_t d, int64_t L_max, int32_t k_max,
                                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * One readout step.
 *   hidden     [L, d] bf16 final hidden states of this step (16-byte aligned)
 *   L          sequence length, 1 <= L <= L_max
 *   mask       [L] u8 in/out: nonzero = position still holds the mask token
 *   tokens     [L] i32 in/out: committed positions receive their argmax token
 *   k          unmask count, 0 <= k <= k_max; n = min(k, M) positions commit
 *   win_lo, win_hi  only positions in [win_lo, win_hi) are candidates
 *              (0 <= win_lo <= win_hi <= L); nothing outside is read or written
 *   block      0: every masked position of the window is a candidate.
 *              > 0: block-wise (semi-autoregressive) decoding -- the window is
 *              cut into blocks of `block` positions starting at win_lo and
 *              only the first block that still holds a masked position
 *              supplies candidates (Sparse-dLLM, Experiment "Memory": logits
 *              only for the current block; 32-token blocks in More Results).
 *   out        host pointer to optional outputs, or NULL
 * M = 0 or k = 0 commits nothing and returns DLLM_OK.
 */
dllm_status dllm_masked_readout_step(dllm_readout *h, const uint16_t *hidden, int64_t L,
                                     uint8_t *mask, int32_t *tokens, int32_t k, int64_t win_lo,
                                     int64_t win_hi, int64_t block, const dllm_step_out *out);

/*
 * One readout step under a selection policy (NULL = top-k by confidence,
 * which is exactly dllm_masked_readout_step).  Arguments as for
 * dllm_masked_readout_step; ties in the score commit the lower position
 * first.  DLLM_ERR_INVALID_ARG for an unknown score, use_threshold not 0 or
 * 1, or a NaN tau.
 */
dllm_status dllm_masked_readout_step_ex(dllm_readout *h, const uint16_t *hidden, int64_t L,
                                        uint8_t *mask, int32_t *tokens, int32_t k, int64_t win_lo,
                                        int64_t win_hi, int64_t block, const dllm_policy *policy,
                                        const dllm_step_out *out);

/* Largest number of sequences one batched step takes. */
#define DLLM_BATCH_MAX 128

/* One sequence of a batched step (host struct). */
typedef struct {
  int32_t k;      /* unmask count of this sequence, 0 <= k <= k_max */
  int32_t win_lo; /* candidate window [win_lo, win_hi) of this sequence, */
  int32_t win_hi; /* 0 <= win_lo <= win_hi <= L                          */
} dllm_seq;

/*
 * Batched readout step: B sequences of length L, decoded together, share one
 * pass over W_lm (serving concurrent requests: Accelerating Masked Diffusion
 * Large Language Models: A Survey of Efficient Inference Techniques, Main
 * Findings, microbatching and throughput-bound serving).  Each sequence gets
 * exactly the result of dllm_masked_readout_step_ex on it alone, with its own
 * k and window; block and policy are common.
 *   B          1 <= B <= DLLM_BATCH_MAX, and B * L <= L_max of the handle
 *   hidden     [B, L, d] bf16 (16-byte aligned)
 *   mask       [B, L] u8 in/out;  tokens [B, L] i32 in/out
 *   seqs       host array [B]
 *   block      as for dllm_masked_readout_step (>= 0)
 *   policy     NULL = top-k by confidence
 *   out        host struct of optional device outputs, now per sequence:
 *              n_out, m_out [B]; sel_idx, sel_tok, sel_conf [B * k_max] with
 *              sequence b at b * k_max; row_* [B * L] with sequence b at
 *              b * L.  Positions are within the sequence (0 <= p < L).
 * Errors as for dllm_masked_readout_step, checked for every sequence before
 * anything is queued.
 */
dllm_status dllm_masked_readout_step_batch(dllm_readout *h, int32_t B, const uint16_t *hidden, int64_t L,
                                           uint8_t *mask, int32_t *tokens, const dllm_seq *seqs,
                                           int64_t block, const dllm_policy *policy,
                                           const dllm_step_out *out);

/* Size of the library's static device scratch, per GPU (see below). */
#define DLLM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * One readout step with no handle and no workspace argument, for callers
 * that cannot allocate device memory or create a workspace: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments and results are those of dllm_masked_readout_create followed by
 * dllm_masked_readout_step_ex with L_max = L and k_max = k (same checks, same
 * kernels, same results).  Instead of a caller workspace the step uses a
 * static device array of DLLM_NOALLOC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends; the call itself allocates
 * nothing (no hipMalloc, no allocating library routine).
 *   stream   hipStream_t to queue the step on (NULL = the default stream);
 *            the call returns without waiting, like dllm_masked_readout_step
 * The first call on a device, with that device current, looks up the
 * array's device address (hipGetSymbolAddress) and keeps it.
 * Limits: DLLM_ERR_WORKSPACE when dllm_masked_readout_workspace_bytes(L, d,
 * V, k) exceeds DLLM_NOALLOC_SCRATCH_BYTES (at V = 126464 about L <= 25000);
 * k <= DLLM_K_MAX_LIMIT.  Nothing is queued on an error.
 * Concurrency: every call on one GPU uses that GPU's one scratch array, and
 * the array keeps the last call's contents (each step writes what it reads
 * first, so stale contents do not matter).  Calls whose work overlaps in
 * time on one GPU -- on different streams or from different host threads --
 * race on the array; queue them on one stream (or otherwise serialise them).
 */
dllm_status dllm_masked_readout_step_noalloc(const uint16_t *W_lm, int64_t V, int64_t d, const uint16_t *hidden,
                                             int64_t L, uint8_t *mask, int32_t *tokens, int32_t k,
                                             int64_t win_lo, int64_t win_hi, int64_t block,
                                             const dllm_policy *policy, const dllm_step_out *out, void *stream);

/* Free the host handle (no device memory is owned).  NULL -> DLLM_OK. */
dllm_status dllm_masked_readout_destroy(dllm_readout *h);

/* Static description of a status code. */
const char *dllm_status_string(dllm_status s);

/*
 * Number of vocabulary slices the compute-bound GEMM path splits V into
 * (each slice yields one partial per row, merged afterwards).  0 = chosen
 * from the window and the device.  Results do not depend on it beyond
 * float32 rounding of the confidence and log-sum-exp.  Exposed for tests
 * and tuning.  DLLM_ERR_INVALID_ARG if slices < 0 or > 64.
 */
dllm_status dllm_masked_readout_set_slices(dllm_readout *h, int32_t slices);

/*
 * Benchmark hook: when both are non-NULL, every later step records
 * ev_before (a hipEvent_t) on the handle's stream right before it queues the
 * GEMM kernel and ev_after right after it, so hipEventElapsedTime gives that
 * kernel's duration.  The events are created and owned by the caller; pass
 * NULL, NULL to stop.  DLLM_ERR_INVALID_ARG if h is NULL or only one event
 * is given.
 */
dllm_status dllm_masked_readout_set_gemm_events(dllm_readout *h, void *ev_before, void *ev_after);

#ifdef __cplusplus
}
#endif
#endif /* DLLM_READOUT_H */
