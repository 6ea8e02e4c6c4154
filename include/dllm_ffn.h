/*
 * dllm_ffn.h -- C ABI of the sequence-chunked SwiGLU FFN of a masked
 * diffusion LLM on AMD Instinct MI355X (gfx950).
 *
 * A dLLM recomputes its activations over the whole sequence at every
 * denoising step, and at low mask ratio the FFN's transient activations --
 * not the logits -- set the memory peak (Mosaic: Unlocking Long-Context
 * Inference for Diffusion LLMs via Global Memory Planning and Dynamic Peak
 * Taming, Abstract and Fig. 3).  Chunking the FFN along the sequence bounds
 * that peak: here the only intermediate is one bf16 [chunk, F] activation.
 *
 * FFN(x) = W_down (SiLU(W_gate x) * (W_up x)),  SiLU(g) = g / (1 + e^-g),
 * for every row x of X (the SwiGLU MLP of LLaMA-family models; the pages give
 * no formula).  bf16 inputs and weights, fp32 accumulation, the activation
 * and the output rounded to bf16 (nearest, ties to even).
 *
 * Memory: every pointer is a DEVICE pointer; bf16 is passed as uint16_t bit
 * patterns; arrays are row-major, contiguous and 16-byte aligned.  The caller
 * owns everything, including the workspace; nothing is allocated.  Work is
 * queued on `stream` (a hipStream_t, NULL = the default stream) and the calls
 * return without waiting.  Argument errors return before anything is queued.
 * The status codes are those of dllm_readout.h.
 */
#ifndef DLLM_FFN_H
#define DLLM_FFN_H

#include <stddef.h>
#include <stdint.h>

#include "dllm_readout.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Bytes of workspace for chunks of `chunk` rows (the bf16 [chunk, F]
 * activation).  0 if chunk < 1 or F < 1.
 */
size_t dllm_ffn_workspace_bytes(int64_t chunk, int64_t F);

/*
 * Pack W_gate [F, d] and W_up [F, d] into W_gu [2F, d], the layout
 * dllm_ffn_swiglu_chunked reads: 64-row units, unit u = gate rows
 * [32u, 32u + 32) followed by up rows [32u, 32u + 32).  One-time weight
 * preparation.  F % 128 == 0 and d % 8 == 0, else DLLM_ERR_UNSUPPORTED.
 */
dllm_status dllm_ffn_pack_gate_up(const uint16_t *W_gate, const uint16_t *W_up, int64_t F, int64_t d,
                                  uint16_t *W_gu, void *stream);

/*
 * Y [L, d] = FFN(X [L, d]), `chunk` rows at a time.
 *   W_gu     [2F, d] packed gate/up weights (dllm_ffn_pack_gate_up)
 *   W_down   [d, F]
 *   chunk    rows per chunk (>= 1); the peak transient is chunk * F * 2 bytes
 *   Y        may be X itself (in place); no other overlap is allowed
 *   workspace  >= dllm_ffn_workspace_bytes(chunk, F) bytes
 * Requirements: d % 256 == 0, F % 128 == 0, and chunk * max(d, F) * 2 < 2^32
 * (DLLM_ERR_UNSUPPORTED otherwise).  L = 0 queues nothing.
 */
dllm_status dllm_ffn_swiglu_chunked(const uint16_t *X, int64_t L, int64_t d, const uint16_t *W_gu,
                                    const uint16_t *W_down, int64_t F, int64_t chunk, uint16_t *Y,
                                    void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DLLM_FFN_H */
