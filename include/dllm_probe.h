/*
 * dllm_probe.h -- measurement aid for the masked-token readout on MI355X:
 * the practical ceiling of its compute-bound LM-head GEMM.
 *
 * The readout's GEMM (Z = H[candidates] . W_lm^T with the fused vocabulary
 * reduction; Mosaic, Unlocking Long-Context Inference for Diffusion LLMs via
 * Global Memory Planning and Dynamic Peak Taming, Abstract: mask-only
 * logits) is bound by the matrix pipes.  How fast those run depends on more
 * than the published dense peak: the sustained clock drops with the bit
 * toggle rate of the operands.  This probe runs the GEMM main loop's
 * instruction mix alone -- one 256-thread workgroup per compute unit, 64
 * v_mfma_f32_32x32x16_bf16 per wave and 64-deep stage, with (mode 1) the
 * loop's 32 fragment loads from LDS, 16 whole-line global->LDS DMAs from an
 * L2-resident region and one barrier -- on operands read from a caller
 * buffer, so that random bf16 data gives the clock the real workload sees.
 * No gather, vocabulary fold or partials: the result bounds what the readout
 * GEMM can reach on this chip.  Flops per call: grid * 4 waves * stages * 64
 * MFMAs * 32768.
 */
#ifndef DLLM_PROBE_H
#define DLLM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "dllm_readout.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the operand source buffer the probe reads (32 MiB). */
size_t dllm_probe_source_bytes(void);

/* Rate of the current device's constant wall clock in kHz (the unit of the
 * second `clocks` value below); 0 if there is no device. */
int64_t dllm_probe_wall_clock_khz(void);

/*
 * Queue one probe kernel on `stream` (NULL = default stream); returns
 * without waiting.
 *   mode    0: MFMAs only; 1: the main loop's full mix (see above)
 *   src     device buffer of dllm_probe_source_bytes() bytes of bf16 values
 *           (random values give the realistic clock), 16-byte aligned
 *   stages  64-deep K stages per workgroup (>= 1)
 *   sink    device float [grid * 256], written (keeps the work live)
 *   grid    workgroups: the compute-unit count for one per CU
 *   clocks  optional device uint64 [2] (NULL = not wanted): the shader-clock
 *           cycles (s_memtime) and the constant-rate wall-clock ticks
 *           (s_memrealtime, hipDeviceAttributeWallClockRate kHz) that wave 0
 *           of workgroup 0 spent in the loop; their ratio is the sustained
 *           shader clock under this load
 * DLLM_ERR_INVALID_ARG for a null pointer, stages < 1, grid < 1 or another
 * mode; DLLM_ERR_UNSUPPORTED for a misaligned src; DLLM_ERR_HIP if the
 * launch fails.
 */
dllm_status dllm_probe_gemm_mix(int32_t mode, const uint16_t *src, int32_t stages, float *sink, int32_t grid,
                                uint64_t *clocks, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DLLM_PROBE_H */
