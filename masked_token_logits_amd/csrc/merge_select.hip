// Cross-slice merge and selection + commit.
//
// Merge: each row's per-slice partials (m_s, a_s, s_s) become
//   m* = max_s m_s,  a* = lowest a_s among slices with m_s = m*,
//   S  = sum_s s_s * exp(m_s - m*),  lse = m* + ln S,  conf = 1 / S,
// i.e. the softmax probability of the argmax token, exp(m* - lse); with the
// extended statistics also the second-largest logit and the entropy
// (online_state.h).  The row gets a 64-bit selection key: its ranking score
// mapped to an order-preserving 32-bit pattern, above (0xFFFFFFFF - row), so
// larger keys mean a larger score and, on equal scores, the lower row --
// the lower position, since rows are in position order.
//
// Select + commit: n rows are committed -- n = min(k, M) for top-k
// (confidence-driven unmasking: Accelerating Masked Diffusion Large Language
// Models: A Survey of Efficient Inference Techniques, Main Findings), or the
// rows whose score clears tau, at least one and at most k (adaptive parallel
// decoding: Dynamic-dLLM, abstract).  The n largest keys are found by an
// MSB-first radix select with 8-bit digits in one workgroup, gathered,
// sorted descending (bitonic, in LDS) and committed: tokens[pos] = argmax
// token, mask[pos] = 0 -- the update set of the step, nothing else is
// written (survey, Main Findings: Delta_t).
#include "readout_internal.h"

#include <math.h>

#include "few_rows.h"
#include "online_state.h"

namespace dllm {
namespace {

__device__ __forceinline__ uint64_t select_key(float score, int row) {
  // + 0.f maps -0 to +0, so equal scores have equal keys
  return ((uint64_t)float_order_key(score + 0.f) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)row);
}

constexpr int kMergeWaves = 4;

// One wave per row: lanes merge strided slices, then a butterfly.
template <bool EXT>
__global__ __launch_bounds__(kMergeWaves * 64) void k_merge(const int32_t* __restrict__ ctr,
                                                          const int32_t* __restrict__ idx, Partials p, int score,
                                                          int32_t* __restrict__ row_tok,
                                                          float* __restrict__ row_conf,
                                                          float* __restrict__ row_lse,
                                                          uint64_t* __restrict__ keys, dllm_step_out o) {
  const int M = ctr[0];
  const int slices = ctr[3];
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (row >= M) return;
  const size_t base = (size_t)row * (size_t)slices;
  RowState r = row_state_empty();
  for (int j = lane; j < slices; j += 64) {
    RowState y;
    y.m = p.m[base + j];
    y.a = p.a[base + j];
    y.s = p.s[base + j];
    y.m2 = EXT ? p.m2[base + j] : -INFINITY;
    y.t = EXT ? p.t[base + j] : 0.f;
    row_merge<EXT>(r, y);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) row_merge<EXT>(r, shfl_xor_state(r, off));
  if (lane == 0) {
    const RowStats st = row_finish<EXT>(r);
    row_tok[row] = r.a;
    row_conf[row] = st.conf;
    row_lse[row] = st.lse;
    keys[row] = select_key(policy_score(st, score), row);
    if (o.row_idx) o.row_idx[row] = idx[row];
    if (o.row_tok) o.row_tok[row] = r.a;
    if (o.row_conf) o.row_conf[row] = st.conf;
    if (o.row_lse) o.row_lse[row] = st.lse;
    if (EXT && o.row_margin) o.row_margin[row] = st.margin;
    if (EXT && o.row_entropy) o.row_entropy[row] = st.entropy;
  }
}

constexpr int kSelThreads = 1024;
constexpr int kSelU = 4;  // keys per thread loaded together in the radix passes

// One workgroup per sequence (a single sequence: one workgroup over all rows).
// The sequence's rows are [start, start + M) of the compacted list; keys hold
// the global row index, positions are idx[row] - pos_base within the sequence.
__global__ __launch_bounds__(kSelThreads) void k_topk_scatter(
    const int32_t* __restrict__ ctr, const int32_t* __restrict__ req, int64_t L, int k_stride, int k_single,
    Policy pol, const uint64_t* __restrict__ keys, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ row_tok, const float* __restrict__ row_conf, const float* __restrict__ row_lse,
    const float* __restrict__ row_margin, const float* __restrict__ row_entropy, uint8_t* __restrict__ mask,
    int32_t* __restrict__ tokens, dllm_step_out o) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t sel[kTopkCap];
  __shared__ int s_digit, s_remaining, s_done, s_count;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  int start, M, k;
  int64_t pos_base;
  if (req) {
    start = req[4 * b];
    M = req[4 * b + 1];
    k = req[4 * b + 2];
    pos_base = (int64_t)b * L;
  } else {
    start = 0;
    M = ctr[0];
    k = k_single;
    pos_base = 0;
  }
  const uint64_t* kb = keys + start;
  if (req) {
    // batched: this sequence's row outputs, from the merged workspace arrays
    for (int i = tid; i < M; i += kSelThreads) {
      const int r = start + i;
      const size_t slot = (size_t)pos_base + (size_t)i;
      if (o.row_idx) o.row_idx[slot] = (int32_t)(idx[r] - pos_base);
      if (o.row_tok) o.row_tok[slot] = row_tok[r];
      if (o.row_conf) o.row_conf[slot] = row_conf[r];
      if (o.row_lse) o.row_lse[slot] = row_lse[r];
      if (o.row_margin && row_margin) o.row_margin[slot] = row_margin[r];
      if (o.row_entropy && row_entropy) o.row_entropy[slot] = row_entropy[r];
    }
  }
  int n = k < M ? k : M;
  if (pol.use_threshold && n > 0) {
    // rows whose score is >= tau: their key's high word is >= tau's pattern
    const uint32_t tk = float_order_key(pol.tau + 0.f);
    if (tid == 0) s_count = 0;
    __syncthreads();
    int c = 0;
    for (int i = tid; i < M; i += kSelThreads) c += (uint32_t)(kb[i] >> 32) >= tk ? 1 : 0;
    if (c) atomicAdd(&s_count, c);
    __syncthreads();
    const int cnt = s_count;
    __syncthreads();
    n = cnt < 1 ? 1 : (cnt < n ? cnt : n);
  }
  if (tid == 0) {
    if (o.n_out) o.n_out[b] = n;
    if (o.m_out) o.m_out[b] = M;
  }
  if (n <= 0) return;
  const size_t sbase = (size_t)b * (size_t)k_stride;

  if (M <= kSelThreads) {
    // Few rows: every thread ranks its key by counting the larger keys (keys
    // are unique), in LDS; no radix passes.
    uint64_t* kl = sel;   // kTopkCap >= kSelThreads
    if (tid < M) kl[tid] = kb[tid];
    __syncthreads();
    if (tid < M) {
      const uint64_t key = kl[tid];
      int rank = 0;
      for (int i = 0; i < M; ++i) rank += kl[i] > key ? 1 : 0;
      if (rank < n) {
        const int row = start + tid;
        const int pos = idx[row];
        const int tok = row_tok[row];
        tokens[pos] = tok;
        mask[pos] = 0;
        if (o.sel_idx) o.sel_idx[sbase + rank] = (int32_t)(pos - pos_base);
        if (o.sel_tok) o.sel_tok[sbase + rank] = tok;
        if (o.sel_conf) o.sel_conf[sbase + rank] = row_conf[row];
      }
    }
    return;
  }

  uint64_t prefix = 0, pmask = 0;
  if (n < M) {
    int remaining = n;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      // kSelU keys per thread in flight before their histogram updates
      for (int base = 0; base < M; base += kSelU * kSelThreads) {
        uint64_t kk[kSelU];
#pragma unroll
        for (int u = 0; u < kSelU; ++u) {
          const int i = base + u * kSelThreads + tid;
          kk[u] = i < M ? kb[i] : 0;  // past M: skipped by the bound check below
        }
#pragma unroll
        for (int u = 0; u < kSelU; ++u)
          if ((kk[u] & pmask) == prefix && base + u * kSelThreads + tid < M)
            atomicAdd(&hist[(kk[u] >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // The digit holding the remaining-th largest key, searched by one
        // wave: lane l holds digits 255 - 4l - j (j = 0..3, descending), a
        // prefix over the lanes gives the keys above each lane's digits, and
        // the one lane where the count crosses `remaining` (1 <= remaining
        // <= keys with this prefix) picks the digit.
        int c4[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c4[j] = (int)hist[255 - 4 * tid - j];
          sum += c4[j];
        }
        int incl = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off);
          if (tid >= off) incl += y;
        }
        const int excl = incl - sum;
        if (excl < remaining && incl >= remaining) {
          int cum = excl, digit = 255 - 4 * tid - 3;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (cum + c4[j] >= remaining) {
              digit = 255 - 4 * tid - j;
              break;
            }
            cum += c4[j];
          }
          s_digit = digit;
          s_remaining = remaining - cum;
          s_done = (s_remaining == (int)hist[digit]) ? 1 : 0;
        }
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
    const uint64_t key = kb[i];
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
    if (key == 0 || row < start || row >= start + M) continue;  // only reachable if fewer than n keys qualified
    const int pos = idx[row];
    const int tok = row_tok[row];
    tokens[pos] = tok;
    mask[pos] = 0;
    if (o.sel_idx) o.sel_idx[sbase + i] = (int32_t)(pos - pos_base);
    if (o.sel_tok) o.sel_tok[sbase + i] = tok;
    if (o.sel_conf) o.sel_conf[sbase + i] = row_conf[row];
  }
}

// Few rows (<= kSmallBM, the semi-autoregressive block), one workgroup per
// candidate row.  The row's per-slice 16-byte (m, a, s, 0) records, written
// by the streaming GEMM into p.m (and its (m2, t) records in p.m2 for the
// extended statistics), are loaded kFinishU per thread at a time without
// branches (an index past the slice count re-reads the last record and is
// merged as empty), merged in each thread, over the wave by a butterfly and
// over the waves in wave order.  Thread 0 finishes the row and writes its
// results to the workspace rows.  Then each workgroup counts itself in on
// ctr[5] (zeroed by whichever kernel wrote ctr this step): thread 0's
// agent-scope release fence orders its row writes before its atomic, and
// the last workgroup's thread 0 acquires before the workgroup reads every
// row back, ranks and commits (few_rows_commit).  One merge round trip on
// kSmallBM CUs instead of the whole merge on one CU.  A batched step
// (req != nullptr) has rows b * L + p.
constexpr int kFinishThreads = 256;
constexpr int kFinishU = 4;
static_assert(kBatchMax <= kFinishThreads && kSmallBM <= kFinishThreads, "one thread per sequence and per row");
static_assert(kTopkCap >= kSelThreads, "few-row ranking keeps the keys in sel[]");
template <bool EXT>
__global__ __launch_bounds__(kFinishThreads) void k_finish_small(int32_t* __restrict__ ctr,
                                                                const int32_t* __restrict__ idx,
                                                                const int32_t* __restrict__ req, int B, int64_t L,
                                                                int k_stride, Partials p, Policy pol, int k,
                                                                uint8_t* __restrict__ mask,
                                                                int32_t* __restrict__ tokens, dllm_step_out o,
                                                                FewRowResults res) {
  __shared__ FewRowSmem sm;
  __shared__ RowState s_wave[kFinishThreads / 64];
  __shared__ int s_last;
  const int M = ctr[0];
  const int slices = ctr[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  if (r < M) {
    const size_t base = (size_t)r * (size_t)slices;
    const float4* rec = reinterpret_cast<const float4*>(p.m) + base;
    const float2* rx = reinterpret_cast<const float2*>(p.m2) + base;
    RowState st = row_state_empty();
    for (int j0 = tid; j0 < slices; j0 += kFinishThreads * kFinishU) {
      float4 a[kFinishU];
      float2 b[kFinishU];
#pragma unroll
      for (int u = 0; u < kFinishU; ++u) {
        int j = j0 + kFinishThreads * u;
        j = j < slices ? j : slices - 1;
        a[u] = rec[j];
        if (EXT) b[u] = rx[j];
      }
#pragma unroll
      for (int u = 0; u < kFinishU; ++u) {
        const bool ok = j0 + kFinishThreads * u < slices;
        RowState y;
        y.m = ok ? a[u].x : -INFINITY;
        y.a = ok ? __float_as_int(a[u].y) : 0x7FFFFFFF;
        y.s = ok ? a[u].z : 0.f;
        y.m2 = (EXT && ok) ? b[u].x : -INFINITY;
        y.t = (EXT && ok) ? b[u].y : 0.f;
        row_merge<EXT>(st, y);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) row_merge<EXT>(st, shfl_xor_state(st, off));
    if (lane == 0) s_wave[wave] = st;
    __syncthreads();
    if (tid == 0) {
#pragma unroll
      for (int w = 1; w < kFinishThreads / 64; ++w) row_merge<EXT>(st, s_wave[w]);
      const RowStats f = row_finish<EXT>(st);
      res.tok[r] = st.a;
      res.conf[r] = f.conf;
      res.lse[r] = f.lse;
      res.margin[r] = f.margin;
      res.entropy[r] = f.entropy;
    }
  }
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const bool last = atomicAdd(ctr + 5, 1) == (int)gridDim.x - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  if (tid < M) {
    RowStats f;
    f.conf = res.conf[tid];
    f.lse = res.lse[tid];
    f.margin = res.margin[tid];
    f.entropy = res.entropy[tid];
    sm.conf[tid] = f.conf;
    sm.lse[tid] = f.lse;
    sm.margin[tid] = f.margin;
    sm.ent[tid] = f.entropy;
    sm.score[tid] = policy_score(f, pol.score) + 0.f;  // -0 -> +0
    sm.tok[tid] = res.tok[tid];
    sm.seq[tid] = req ? (int)(idx[tid] / L) : 0;
  }
  few_rows_commit<EXT>(sm, M, idx, req, B, L, k_stride, pol, k, mask, tokens, o);
}

}  // namespace

hipError_t launch_finish_small(int32_t* ctr, const int32_t* idx, const int32_t* req, int B, int64_t L, int k_stride,
                               Partials p, Policy pol, int k, uint8_t* mask, int32_t* tokens, dllm_step_out out,
                               FewRowResults res, hipStream_t stream) {
  if (p.ext)
    hipLaunchKernelGGL(k_finish_small<true>, dim3(kSmallBM), dim3(kFinishThreads), 0, stream, ctr, idx, req, B, L,
                       k_stride, p, pol, k, mask, tokens, out, res);
  else
    hipLaunchKernelGGL(k_finish_small<false>, dim3(kSmallBM), dim3(kFinishThreads), 0, stream, ctr, idx, req, B, L,
                       k_stride, p, pol, k, mask, tokens, out, res);
  return hipGetLastError();
}

hipError_t launch_merge(const int32_t* ctr, const int32_t* idx, Partials p, int score, int max_rows,
                        int32_t* row_tok, float* row_conf, float* row_lse, uint64_t* keys,
                        const dllm_step_out& out, hipStream_t stream) {
  const int grid = (max_rows + kMergeWaves - 1) / kMergeWaves;
  if (grid <= 0) return hipSuccess;
  if (p.ext)
    hipLaunchKernelGGL(k_merge<true>, dim3(grid), dim3(kMergeWaves * 64), 0, stream, ctr, idx, p, score, row_tok,
                       row_conf, row_lse, keys, out);
  else
    hipLaunchKernelGGL(k_merge<false>, dim3(grid), dim3(kMergeWaves * 64), 0, stream, ctr, idx, p, score, row_tok,
                       row_conf, row_lse, keys, out);
  return hipGetLastError();
}

hipError_t launch_topk_scatter(const int32_t* ctr, const int32_t* req, int B, int64_t L, int k_stride, int k,
                               Policy pol, const Workspace& ws, uint8_t* mask, int32_t* tokens,
                               const dllm_step_out& out, hipStream_t stream) {
  const int grid = req ? B : 1;
  hipLaunchKernelGGL(k_topk_scatter, dim3(grid), dim3(kSelThreads), 0, stream, ctr, req, L, k_stride, k, pol, ws.keys,
                     ws.idx, ws.row_tok, ws.row_conf, ws.row_lse, ws.row_margin, ws.row_entropy, mask, tokens, out);
  return hipGetLastError();
}

}  // namespace dllm
