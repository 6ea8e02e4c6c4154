// Cross-slice merge and top-k commit.
//
// Merge: each row's per-slice partials (m_s, a_s, s_s) become
//   m* = max_s m_s,  a* = lowest a_s among slices with m_s = m*,
//   S  = sum_s s_s * exp(m_s - m*),  lse = m* + ln S,  conf = 1 / S,
// i.e. the softmax probability of the argmax token, exp(m* - lse).  The row
// also gets a 64-bit selection key: conf's float bits (positive floats order
// like their bit patterns) above (0xFFFFFFFF - row), so larger keys mean
// higher confidence and, on equal confidence, the lower row -- the lower
// position, since rows are in position order.
//
// Select + commit: the n = min(k, M) largest keys (confidence-driven
// unmasking: Accelerating Masked Diffusion Large Language Models: A Survey of
// Efficient Inference Techniques, Main Findings) are found by an MSB-first
// radix select with 8-bit digits in one workgroup, gathered, sorted
// descending (bitonic, in LDS) and committed: tokens[pos] = argmax token,
// mask[pos] = 0 -- the update set of the step, nothing else is written
// (survey, Main Findings: Delta_t).
#include "readout_internal.h"

#include <math.h>

namespace dllm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ void merge_state(float& m, int& a, float& s, float m2, int a2, float s2) {
  const bool take2 = (m2 > m) || (m2 == m && a2 < a);
  const float mn = fmaxf(m, m2);
  const float e1 = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m - mn) * kLog2e);
  const float e2 = (m2 == -INFINITY) ? 0.f : s2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
  a = take2 ? a2 : a;
  m = mn;
  s = e1 + e2;
}

constexpr int kMergeWaves = 4;

__global__ __launch_bounds__(kMergeWaves * 64) void k_merge(
    const int32_t* __restrict__ ctr, const int32_t* __restrict__ idx, const float* __restrict__ pm,
    const int32_t* __restrict__ pa, const float* __restrict__ ps,
    int32_t* __restrict__ row_tok, float* __restrict__ row_conf, float* __restrict__ row_lse,
    uint64_t* __restrict__ keys, int32_t* o_row_idx, int32_t* o_row_tok, float* o_row_conf,
    float* o_row_lse) {
  const int M = ctr[0];
  const int slices = ctr[3];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (row >= M) return;
  const size_t base = (size_t)row * (size_t)slices;
  float m = -INFINITY, s = 0.f;
  int a = 0x7FFFFFFF;
  for (int j = lane; j < slices; j += 64) merge_state(m, a, s, pm[base + j], pa[base + j], ps[base + j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const int a2 = __shfl_xor(a, off);
    const float s2 = __shfl_xor(s, off);
    merge_state(m, a, s, m2, a2, s2);
  }
  if (lane == 0) {
    const float conf = 1.0f / s;
    const float lse = m + __builtin_amdgcn_logf(s) * kLn2;
    row_tok[row] = a;
    row_conf[row] = conf;
    row_lse[row] = lse;
    keys[row] = ((uint64_t)__float_as_uint(conf) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)row);
    if (o_row_idx) o_row_idx[row] = idx[row];
    if (o_row_tok) o_row_tok[row] = a;
    if (o_row_conf) o_row_conf[row] = conf;
    if (o_row_lse) o_row_lse[row] = lse;
  }
}

constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(kSelThreads) void k_topk_scatter(
    const int32_t* __restrict__ ctr, int k, const uint64_t* __restrict__ keys,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ row_tok, uint8_t* __restrict__ mask,
    int32_t* __restrict__ tokens, int32_t* n_out, int32_t* m_out, int32_t* sel_idx, int32_t* sel_tok,
    float* sel_conf) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t sel[kTopkCap];
  __shared__ int s_digit, s_remaining, s_done, s_count;
  const int tid = threadIdx.x;
  const int M = ctr[0];
  const int n = k < M ? k : M;
  if (tid == 0) {
    if (n_out) *n_out = n;
    if (m_out) *m_out = M;
  }
  if (n <= 0) return;

  uint64_t prefix = 0, pmask = 0;
  if (n < M) {
    int remaining = n;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < M; i += kSelThreads) {
        const uint64_t key = keys[i];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int cum = 0, digit = 0;
        for (int dg = 255; dg >= 0; --dg) {
          const int c = (int)hist[dg];
          if (cum + c >= remaining) {
            digit = dg;
            break;
          }
          cum += c;
        }
        s_digit = digit;
        s_remaining = remaining - cum;
        s_done = (s_remaining == (int)hist[digit]) ? 1 : 0;
      }
      __syncthreads();
      prefix |= (uint64_t)s_digit << shift;
      pmask |= (uint64_t)0xFF << shift;
      remaining = s_remaining;
      const int done = s_done;
      __syncthreads();
      if (done) break;
    }
  }
  // Keys are unique (the low word is the row), so exactly n keys are >= prefix.
  if (tid == 0) s_count = 0;
  __syncthreads();
  for (int i = tid; i < M; i += kSelThreads) {
    const uint64_t key = keys[i];
    if (key >= prefix) {
      const int slot = atomicAdd(&s_count, 1);
      if (slot < kTopkCap) sel[slot] = key;
    }
  }
  __syncthreads();
  int P = 1;
  while (P < n) P <<= 1;
  const int got = s_count < n ? s_count : n;
  for (int i = got + tid; i < P; i += kSelThreads) sel[i] = 0;
  __syncthreads();
  // Bitonic sort, descending.
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P; i += kSelThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;
          const uint64_t x = sel[i], y = sel[j];
          if ((x < y) == desc) {
            sel[i] = y;
            sel[j] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < n; i += kSelThreads) {
    const uint64_t key = sel[i];
    const int row = (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
    if (key == 0 || row < 0 || row >= M) continue;  // only reachable if fewer than n keys qualified
    const int pos = idx[row];
    const int tok = row_tok[row];
    tokens[pos] = tok;
    mask[pos] = 0;
    if (sel_idx) sel_idx[i] = pos;
    if (sel_tok) sel_tok[i] = tok;
    if (sel_conf) sel_conf[i] = __uint_as_float((uint32_t)(key >> 32));
  }
}

// Few rows (<= kSmallBM, the semi-autoregressive block): one workgroup
// merges every row's slices (16-byte (m, a, s, 0) records written by the
// streaming GEMM into pm; 32 lanes per row, loads issued 16 at a time
// so their latencies overlap, then a butterfly), ranks the rows by counting
// (row r precedes r' iff its confidence is larger, or equal with the lower
// row = lower position) and commits the first n = min(k, M).
constexpr int kFinishThreads = 1024;
static_assert(kFinishThreads == 32 * kSmallBM, "32 lanes per row");
__global__ __launch_bounds__(kFinishThreads) void k_finish_small(const int32_t* __restrict__ ctr,
                                                                const int32_t* __restrict__ idx,
                                                                const float* __restrict__ pm,
                                                                const int32_t* __restrict__ pa,
                                                                const float* __restrict__ ps, int k,
                                                                uint8_t* __restrict__ mask,
                                                                int32_t* __restrict__ tokens, dllm_step_out o) {
  __shared__ float s_conf[kSmallBM], s_lse[kSmallBM];
  __shared__ int s_tok[kSmallBM];
  const int M = ctr[0];
  const int slices = ctr[3];
  const int r = threadIdx.x >> 5, sub = threadIdx.x & 31;
  if (r < M) {
    const size_t base = (size_t)r * (size_t)slices;
    float m = -INFINITY, s = 0.f;
    int a = 0x7FFFFFFF;
    constexpr int U = 16;
    for (int j0 = sub; j0 < slices; j0 += 32 * U) {
      float mu[U], su[U];
      int au[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + 32 * u;
        float4 rec = make_float4(-INFINITY, __int_as_float(0x7FFFFFFF), 0.f, 0.f);
        if (j < slices) rec = reinterpret_cast<const float4*>(pm)[base + j];
        mu[u] = rec.x;
        au[u] = __float_as_int(rec.y);
        su[u] = rec.z;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) merge_state(m, a, s, mu[u], au[u], su[u]);
    }
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {  // within the 32-lane half of the wave
      const float m2 = __shfl_xor(m, off);
      const int a2 = __shfl_xor(a, off);
      const float s2 = __shfl_xor(s, off);
      merge_state(m, a, s, m2, a2, s2);
    }
    if (sub == 0) {
      s_conf[r] = 1.0f / s;
      s_lse[r] = m + __builtin_amdgcn_logf(s) * kLn2;
      s_tok[r] = a;
    }
  }
  __syncthreads();
  const int n = k < M ? k : M;
  const int t = threadIdx.x;
  if (t < M) {
    const float c = s_conf[t];
    int rank = 0;
    for (int r2 = 0; r2 < M; ++r2) {
      const float c2 = s_conf[r2];
      rank += (c2 > c || (c2 == c && r2 < t)) ? 1 : 0;
    }
    const int pos = idx[t];
    const int tok = s_tok[t];
    if (o.row_idx) o.row_idx[t] = pos;
    if (o.row_tok) o.row_tok[t] = tok;
    if (o.row_conf) o.row_conf[t] = c;
    if (o.row_lse) o.row_lse[t] = s_lse[t];
    if (rank < n) {
      tokens[pos] = tok;
      mask[pos] = 0;
      if (o.sel_idx) o.sel_idx[rank] = pos;
      if (o.sel_tok) o.sel_tok[rank] = tok;
      if (o.sel_conf) o.sel_conf[rank] = c;
    }
  }
  if (t == 0) {
    if (o.n_out) *o.n_out = n;
    if (o.m_out) *o.m_out = M;
  }
}

}  // namespace

hipError_t launch_finish_small(const int32_t* ctr, const int32_t* idx, const float* pm, const int32_t* pa,
                               const float* ps, int k, uint8_t* mask, int32_t* tokens, dllm_step_out out,
                               hipStream_t stream) {
  hipLaunchKernelGGL(k_finish_small, dim3(1), dim3(kFinishThreads), 0, stream, ctr, idx, pm, pa, ps, k, mask, tokens,
                     out);
  return hipGetLastError();
}

hipError_t launch_merge(const int32_t* ctr, const int32_t* idx, const float* pm, const int32_t* pa,
                        const float* ps, int max_rows, int32_t* row_tok, float* row_conf,
                        float* row_lse, uint64_t* keys, int32_t* o_row_idx, int32_t* o_row_tok,
                        float* o_row_conf, float* o_row_lse, hipStream_t stream) {
  const int grid = (max_rows + kMergeWaves - 1) / kMergeWaves;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_merge, dim3(grid), dim3(kMergeWaves * 64), 0, stream, ctr, idx, pm, pa, ps,
                     row_tok, row_conf, row_lse, keys, o_row_idx, o_row_tok, o_row_conf, o_row_lse);
  return hipGetLastError();
}

hipError_t launch_topk_scatter(const int32_t* ctr, int k, const uint64_t* keys, const int32_t* idx,
                               const int32_t* row_tok, uint8_t* mask, int32_t* tokens,
                               int32_t* n_out, int32_t* m_out, int32_t* sel_idx, int32_t* sel_tok,
                               float* sel_conf, hipStream_t stream) {
  hipLaunchKernelGGL(k_topk_scatter, dim3(1), dim3(kSelThreads), 0, stream, ctr, k, keys, idx, row_tok,
                     mask, tokens, n_out, m_out, sel_idx, sel_tok, sel_conf);
  return hipGetLastError();
}

}  // namespace dllm
