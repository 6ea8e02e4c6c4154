// Internal declarations shared by the host library and the kernels of the
// masked-token readout (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dllm_readout.h"

namespace dllm {

// Layout of the device workspace, carved by the host at create time.
struct Workspace {
  int32_t* idx;        // [L_max]   candidate positions, ascending (compaction output)
  int32_t* ctr;        // [16]      ctr[0] = M, ctr[1] = lo, ctr[2] = hi of the candidate window,
                       //           ctr[3] = vocabulary slices S of this step, ctr[4] = row tiles,
                       //           ctr[5] = arrivals of the few-row finish (zeroed with ctr[0..4])
  float* part_m;       // [part_cap] per (row, slice) running max logit
  int32_t* part_a;     // [part_cap] per (row, slice) argmax vocabulary index
  float* part_s;       // [part_cap] per (row, slice) sum of exp(z - part_m)
  float* part_m2;      // [part_cap] extended statistics: second-largest logit
  float* part_t;       // [part_cap] extended statistics: sum exp(z - part_m) * (z - part_m)
  int32_t* row_tok;    // [L_max]   merged argmax per candidate row
  float* row_conf;     // [L_max]   merged confidence
  float* row_lse;      // [L_max]   merged log-sum-exp
  uint64_t* keys;      // [L_max]   selection key: ordered score bits << 32 | (0xFFFFFFFF - row)
  float* row_margin;   // [L_max]   merged margin (batched steps with the extended statistics)
  float* row_entropy;  // [L_max]   merged entropy (same)
  int32_t* req;        // [4 * kBatchMax] per sequence of a batched step: first row, M, k, 0
  int64_t part_cap;
};

constexpr int kBatchMax = DLLM_BATCH_MAX;

// The sequences of a batched step, passed by value to the compaction kernel
// (1.5 KiB of kernel arguments), which records them in Workspace::req.
struct SeqTable {
  int32_t lo[kBatchMax], hi[kBatchMax], k[kBatchMax];
};

// Partials of one step: (m, a, s) always, (m2, t) when `ext` (margin or
// entropy requested).  The few-row path stores (m, a, s, 0) float4 records
// in m and (m2, t) float2 records in m2.
struct Partials {
  float* m;
  int32_t* a;
  float* s;
  float* m2;
  float* t;
  bool ext;
};

// Selection policy as the kernels see it (validated dllm_policy).
struct Policy {
  int score;          // 0 conf, 1 margin, 2 negative entropy
  int use_threshold;  // 0 top-k, 1 threshold with cap k
  float tau;
};

// Tile shapes of the two GEMM variants (rows = candidate rows, vocab = W_lm rows).
constexpr int kBK = 64;                 // K elements per LDS stage
constexpr int kLargeBM = 256, kLargeBN = 256;
constexpr int kSmallBM = 32, kSmallBN = 128;
constexpr int kMaxLargeSlices = 64;
constexpr int kMaxSmallSlices = 2048;
constexpr int kTopkCap = 4096;          // largest k the selection kernel holds in LDS

// How the step's work is split, decided on the device once M is known.
//   fixed_slices > 0: S = fixed_slices (rows are one tile of `tile_rows`).
//   fixed_slices == 0: persistent GEMM with `grid` workgroups; S is chosen
//   so that the n_rt * S (row tile, slice) items fill whole rounds of the
//   grid with equally long items, with n_rt * tile_rows * S <= part_cap.
struct PlanParams {
  int fixed_slices;
  int tile_rows;
  int n_vt;        // vocabulary tiles
  int grid;        // persistent workgroups
  int max_slices;
  int64_t part_cap;
};

// Kernel launchers (each queues exactly one kernel on `stream`).
hipError_t launch_mask_compact(const uint8_t* mask, int64_t win_lo, int64_t win_hi, int64_t block,
                               PlanParams plan, int32_t* idx, int32_t* ctr, hipStream_t stream);

// Batched: B windows, one per sequence of length L (rows are b * L + p);
// writes Workspace::req and the plan for the total M.
hipError_t launch_mask_compact_batch(const uint8_t* mask, int B, int64_t L, const SeqTable& seqs, int64_t block,
                                     PlanParams plan, int32_t* idx, int32_t* ctr, int32_t* req, hipStream_t stream);

// The same for windows that hold at most 32 candidates (one wave).
hipError_t launch_mask_compact_small(const uint8_t* mask, int64_t win_lo, int64_t win_hi, int64_t block,
                                     int fixed_slices, int32_t* idx, int32_t* ctr, hipStream_t stream);

hipError_t launch_gemm_large(const uint16_t* W, const uint16_t* H, int d, int V, const int32_t* idx,
                             const int32_t* ctr, int n_row_tiles, int slices, Partials p, hipStream_t stream);

// Persistent compute-bound variant (d % 32 == 0): `grid` workgroups walk the
// (row tile, slice) items of the device-side plan in ctr[3], ctr[4].  With
// d % kPersistWideBK == 0 its main loop runs 64-deep stages of whole
// 128-byte lines; otherwise 32-deep stages of half lines.
constexpr int kPersistBM = 256, kPersistBN = 256, kPersistBK = 32, kPersistStages = 4;
constexpr int kPersistWideBK = 64;
hipError_t launch_gemm_persistent(const uint16_t* W, const uint16_t* H, int d, int V, const int32_t* idx,
                                  const int32_t* ctr, int grid, Partials p, hipStream_t stream);

// The persistent GEMM's store epilogues (FFN): out[M, ldo] (bf16) = X[M, K] . W^T,
// W [n_w_rows, K]; n_w_rows % 256 == 0.  swiglu: W holds gate/up rows in
// 64-row units (32 gate rows, then the 32 up rows of the same outputs) and
// out gets SiLU(gate) * up, n_w_rows / 2 columns.
constexpr int kEpiReadout = 0, kEpiStore = 1, kEpiSwiGLU = 2;
struct StoreArgs {
  uint16_t* out;
  int ldo;
  int M;
};
hipError_t launch_gemm_store(bool swiglu, const uint16_t* W, int n_w_rows, const uint16_t* X, int K, int M,
                             uint16_t* out, int ldo, int grid, hipStream_t stream);

// The candidate search of a single-sequence few-row step, done by the GEMM
// itself (every workgroup finds the same rows; workgroup 0 writes the list
// to idx and M, lo, hi, slices, 1, 0 to ctr[0..5] for the finish, as the
// compaction kernel would).
struct FindRows {
  const uint8_t* mask;
  int64_t win_lo, win_hi, block;
  int32_t* idx;
  int32_t* ctr;
};

// Few-row GEMM.  find == nullptr: rows from the compaction (idx, ctr).
hipError_t launch_gemm_small(const uint16_t* W, const uint16_t* H, int d, int V, const int32_t* idx,
                             const int32_t* ctr, int slices, Partials p, const FindRows* find, hipStream_t stream);

// Per-row results of the few-row finish (workspace rows, kSmallBM used).
struct FewRowResults {
  int32_t* tok;
  float* conf;
  float* lse;
  float* margin;
  float* entropy;
};

// Merge + selection + commit for at most kSmallBM candidate rows: one
// workgroup per row, the last one to finish commits (counts on ctr[5], which
// the kernel that wrote ctr this step has zeroed).  Replaces launch_merge +
// launch_topk_scatter on the small path.  Batched (req != nullptr): B
// sequences of length L, each ranked on its own; outputs per sequence at
// b * k_stride (selection) and b * L (rows).
hipError_t launch_finish_small(int32_t* ctr, const int32_t* idx, const int32_t* req, int B, int64_t L, int k_stride,
                               Partials p, Policy pol, int k, uint8_t* mask, int32_t* tokens, dllm_step_out out,
                               FewRowResults res, hipStream_t stream);

hipError_t launch_merge(const int32_t* ctr, const int32_t* idx, Partials p, int score, int max_rows,
                        int32_t* row_tok, float* row_conf, float* row_lse, uint64_t* keys,
                        const dllm_step_out& out, hipStream_t stream);

// Selection + commit.  Single sequence (req == nullptr): one workgroup over
// all M rows, k as given; the merge already wrote the row outputs.
// Batched: one workgroup per sequence over its rows (Workspace::req), which
// also copies the sequence's row outputs from the workspace arrays.
hipError_t launch_topk_scatter(const int32_t* ctr, const int32_t* req, int B, int64_t L, int k_stride, int k,
                               Policy pol, const Workspace& ws, uint8_t* mask, int32_t* tokens,
                               const dllm_step_out& out, hipStream_t stream);

}  // namespace dllm
