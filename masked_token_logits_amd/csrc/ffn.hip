// Host side of the sequence-chunked SwiGLU FFN (include/dllm_ffn.h) and the
// gate/up weight packing kernel.  Each chunk of rows is two launches of the
// persistent MFMA GEMM: X_chunk . W_gu^T with the SwiGLU epilogue into the
// bf16 [chunk, F] activation, then activation . W_down^T with the bf16 store
// epilogue into Y's rows.  The chunk's activation is the only intermediate,
// so the FFN's transient memory is chunk * F * 2 bytes instead of the
// L * F-sized gate, up and activation tensors (Mosaic, Fig. 3: the FFN peak
// at low mask ratio).
#include "dllm_ffn.h"
#include "readout_internal.h"

namespace dllm {
namespace {

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

// Packed row R of W_gu is gate row 32 (R / 64) + R % 32 for R % 64 < 32, else
// that up row; one thread per 16-byte chunk.
__global__ __launch_bounds__(256) void k_pack_gate_up(const uint16_t* __restrict__ Wg,
                                                      const uint16_t* __restrict__ Wu, int64_t F, int64_t d,
                                                      uint16_t* __restrict__ Wgu) {
  const int64_t cpr = d / 8;  // 16-byte chunks per row
  const int64_t n = 2 * F * cpr;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t R = t / cpr, c = t - R * cpr;
    const int64_t src_row = 32 * (R / 64) + (R & 31);
    const uint16_t* src = ((R & 63) < 32 ? Wg : Wu) + src_row * d + c * 8;
    *reinterpret_cast<u32x4*>(Wgu + R * d + c * 8) = *reinterpret_cast<const u32x4*>(src);
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

}  // namespace
}  // namespace dllm

extern "C" {

size_t dllm_ffn_workspace_bytes(int64_t chunk, int64_t F) {
  if (chunk < 1 || F < 1 || chunk > ((int64_t)1 << 31) || F > ((int64_t)1 << 31)) return 0;
  return (size_t)chunk * (size_t)F * sizeof(uint16_t);
}

dllm_status dllm_ffn_pack_gate_up(const uint16_t* W_gate, const uint16_t* W_up, int64_t F, int64_t d,
                                  uint16_t* W_gu, void* stream) {
  if (!W_gate || !W_up || !W_gu || F < 1 || d < 1) return DLLM_ERR_INVALID_ARG;
  if (F % 128 != 0 || d % 8 != 0) return DLLM_ERR_UNSUPPORTED;
  if (!dllm::aligned16(W_gate) || !dllm::aligned16(W_up) || !dllm::aligned16(W_gu)) return DLLM_ERR_UNSUPPORTED;
  const int64_t n = 2 * F * (d / 8);
  const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
  hipLaunchKernelGGL(dllm::k_pack_gate_up, dim3((unsigned)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), W_gate, W_up, F, d, W_gu);
  return hipGetLastError() == hipSuccess ? DLLM_OK : DLLM_ERR_HIP;
}

dllm_status dllm_ffn_swiglu_chunked(const uint16_t* X, int64_t L, int64_t d, const uint16_t* W_gu,
                                    const uint16_t* W_down, int64_t F, int64_t chunk, uint16_t* Y,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!X || !W_gu || !W_down || !Y) return DLLM_ERR_INVALID_ARG;
  if (L < 0 || L >= ((int64_t)1 << 31) || d < 1 || F < 1 || chunk < 1) return DLLM_ERR_INVALID_ARG;
  if (d % 256 != 0 || F % 128 != 0) return DLLM_ERR_UNSUPPORTED;
  const int64_t wide = d > F ? d : F;
  // the persistent GEMM uses 32-bit byte offsets for the rows of a chunk and of a 256-row weight tile
  if (chunk * wide * 2 >= ((int64_t)1 << 32) || 256 * wide * 2 >= ((int64_t)1 << 32)) return DLLM_ERR_UNSUPPORTED;
  if (!dllm::aligned16(X) || !dllm::aligned16(W_gu) || !dllm::aligned16(W_down) || !dllm::aligned16(Y))
    return DLLM_ERR_UNSUPPORTED;
  const size_t need = dllm_ffn_workspace_bytes(chunk, F);
  if (!workspace || workspace_bytes < need || !dllm::aligned16(workspace)) return DLLM_ERR_WORKSPACE;
  if (L == 0) return DLLM_OK;
  const int cus = dllm::device_cus();
  if (cus <= 0) return DLLM_ERR_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint16_t* act = reinterpret_cast<uint16_t*>(workspace);
  for (int64_t r0 = 0; r0 < L; r0 += chunk) {
    const int rows = (int)(L - r0 < chunk ? L - r0 : chunk);
    // activation [rows, F] = SiLU(X W_gate^T) * (X W_up^T)
    if (dllm::launch_gemm_store(true, W_gu, (int)(2 * F), X + r0 * d, (int)d, rows, act, (int)F, cus, st) !=
        hipSuccess)
      return DLLM_ERR_HIP;
    // Y rows [r0, r0 + rows) = activation W_down^T
    if (dllm::launch_gemm_store(false, W_down, (int)d, act, (int)F, rows, Y + r0 * d, (int)d, cus, st) != hipSuccess)
      return DLLM_ERR_HIP;
  }
  return DLLM_OK;
}

}  // extern "C"
