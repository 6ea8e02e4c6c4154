// Internal declarations shared by the host library and the kernels of the
// masked-token readout (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dllm {

// Layout of the device workspace, carved by the host at create time.
struct Workspace {
  int32_t* idx;        // [L_max]   candidate positions, ascending (compaction output)
  int32_t* ctr;        // [16]      ctr[0] = M, ctr[1] = lo, ctr[2] = hi of the candidate window
  float* part_m;       // [part_cap] per (row, slice) running max logit
  int32_t* part_a;     // [part_cap] per (row, slice) argmax vocabulary index
  float* part_s;       // [part_cap] per (row, slice) sum of exp(z - part_m)
  int32_t* row_tok;    // [L_max]   merged argmax per candidate row
  float* row_conf;     // [L_max]   merged confidence
  float* row_lse;      // [L_max]   merged log-sum-exp
  uint64_t* keys;      // [L_max]   selection key: conf bits << 32 | (0xFFFFFFFF - row)
  int64_t part_cap;
};

// Tile shapes of the two GEMM variants (rows = candidate rows, vocab = W_lm rows).
constexpr int kBK = 64;                 // K elements per LDS stage
constexpr int kLargeBM = 256, kLargeBN = 256;
constexpr int kSmallBM = 32, kSmallBN = 128;
constexpr int kMaxLargeSlices = 64;
constexpr int kMaxSmallSlices = 2048;
constexpr int kTopkCap = 4096;          // largest k the selection kernel holds in LDS

// Kernel launchers (each queues exactly one kernel on `stream`).
hipError_t launch_mask_compact(const uint8_t* mask, int64_t win_lo, int64_t win_hi, int64_t block,
                               int32_t* idx, int32_t* ctr, hipStream_t stream);

hipError_t launch_gemm_large(const uint16_t* W, const uint16_t* H, int d, int V, const int32_t* idx,
                             const int32_t* ctr, int n_row_tiles, int slices, float* pm, int32_t* pa,
                             float* ps, hipStream_t stream);

hipError_t launch_gemm_small(const uint16_t* W, const uint16_t* H, int d, int V, const int32_t* idx,
                             const int32_t* ctr, int slices, float* pm, int32_t* pa, float* ps,
                             hipStream_t stream);

hipError_t launch_merge(const int32_t* ctr, const int32_t* idx, const float* pm, const int32_t* pa,
                        const float* ps, int slices, int max_rows, int32_t* row_tok, float* row_conf,
                        float* row_lse, uint64_t* keys, int32_t* o_row_idx, int32_t* o_row_tok,
                        float* o_row_conf, float* o_row_lse, hipStream_t stream);

hipError_t launch_topk_scatter(const int32_t* ctr, int k, const uint64_t* keys, const int32_t* idx,
                               const int32_t* row_tok, uint8_t* mask, int32_t* tokens,
                               int32_t* n_out, int32_t* m_out, int32_t* sel_idx, int32_t* sel_tok,
                               float* sel_conf, hipStream_t stream);

}  // namespace dllm
