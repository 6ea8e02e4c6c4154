// Mask compaction: the ascending list of positions that still hold the mask
// token inside the step's window ("mask-only logits", Mosaic Abstract), and
// for block-wise decoding the first block of the window that still holds
// one (Sparse-dLLM, Experiment "Memory": logits only for the current block).
//
// One workgroup of 1024 threads walks the window in chunks of 16 Ki
// positions; each thread owns 16 consecutive mask bytes.  Within a wavefront
// the exclusive prefix of the per-thread counts comes from ballots of the
// count's bits (count = sum_b 2^b * bit_b, so the prefix is
// sum_b 2^b * popcount(ballot(bit_b) & lanes-below)), across the 16 waves
// from a small LDS table.  Each chunk's positions are placed in LDS at
// those offsets and stored to idx as one contiguous run.  M and the window
// actually used go to ctr[0..2] so no host synchronisation is needed before
// the next kernel.
//
// The same kernel then fixes how the GEMM splits the work, now that M is
// known (choose_plan).  A batched step compacts every sequence's window
// into one list of rows (k_mask_compact_batch).
#include "few_rows.h"
#include "readout_internal.h"

namespace dllm {
namespace {

constexpr int kThreads = 1024;
constexpr int kPerThread = 16;
constexpr int kChunk = kThreads * kPerThread;
static_assert(kPerThread == 16, "mask_bits16 covers 16 positions");

// Work plan once M is known (every thread of the workgroup calls this):
// fixed slices, or for the persistent GEMM the slice count S minimising
// (rounds of the grid) x (longest item), one candidate per thread (ties:
// fewer slices).  The candidates' keys (cost << 20 | S) are reduced within
// each wave first, so one LDS atomicMin per wave remains, and the per-thread
// arithmetic is 32-bit: a candidate that passes the workspace check has
// n_rt * S * tile_rows <= part_cap, so n_rt * S < 2^29 here.
__device__ void choose_plan(int M, const PlanParams& plan, unsigned long long* s_best, int& S, int& n_rt) {
  const int tid = threadIdx.x;
  n_rt = (M + plan.tile_rows - 1) / plan.tile_rows;
  S = plan.fixed_slices;
  if (S > 0) return;
  if (tid == 0) *s_best = ~0ull;
  __syncthreads();
  unsigned long long key = ~0ull;
  if (n_rt > 0) {
    for (int c = tid + 1; c <= plan.max_slices && c <= plan.n_vt; c += blockDim.x) {
      if ((int64_t)n_rt * plan.tile_rows * c > plan.part_cap) break;
      const unsigned items = (unsigned)n_rt * (unsigned)c;
      const unsigned rounds = (items + (unsigned)plan.grid - 1u) / (unsigned)plan.grid;
      const unsigned len = ((unsigned)plan.n_vt + (unsigned)c - 1u) / (unsigned)c;  // vocabulary tiles of the longest item
      const unsigned long long cost = (unsigned long long)rounds * (4ull * len + 1ull);
      const unsigned long long k = (cost << 20) | (unsigned long long)c;
      key = k < key ? k : key;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = (unsigned long long)__shfl_xor((long long)key, off);
    key = o < key ? o : key;
  }
  if ((tid & 63) == 0 && key != ~0ull) atomicMin(s_best, key);
  __syncthreads();
  S = (*s_best == ~0ull) ? 1 : (int)(*s_best & 0xFFFFF);
}

// ---- one-wave building blocks of the batched compaction -------------------
// Lanes cover 16 consecutive mask bytes each, 1024 positions per pass.

// Block mode: narrow [lo, hi) to the first `block`-aligned block (counted
// from the window start) that still holds a masked position; empty if none.
__device__ void wave_block_window(const uint8_t* __restrict__ m, int64_t block, int& lo, int& hi) {
  const int lane = threadIdx.x & 63;
  int first = hi;
  for (int base = lo; base < hi; base += 64 * 16) {
    const int p0 = base + lane * 16;
    const unsigned bits = p0 < hi ? mask_bits16(m, p0, hi) : 0u;
    const int mine = bits ? p0 + __ffs(bits) - 1 : hi;
    const unsigned long long bal = __ballot(mine < hi);  // lanes cover increasing positions
    if (bal) {
      first = __shfl(mine, __ffsll((long long)bal) - 1);
      break;
    }
  }
  if (first >= hi) {
    lo = hi;
  } else {
    const int64_t blo = (int64_t)lo + (int64_t)((first - lo) / block) * block;
    const int64_t bhi = blo + block < (int64_t)hi ? blo + block : (int64_t)hi;
    lo = (int)blo;
    hi = (int)bhi;
  }
}

// Number of masked positions in [lo, hi) (the same value in every lane).
__device__ int wave_count(const uint8_t* __restrict__ m, int lo, int hi) {
  const int lane = threadIdx.x & 63;
  int c = 0;
  for (int base = lo; base < hi; base += 64 * 16) {
    const int p0 = base + lane * 16;
    c += p0 < hi ? __popc(mask_bits16(m, p0, hi)) : 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
  return c;
}

// Write row_base + p for every masked p in [lo, hi), ascending, to out[0..).
__device__ void wave_write(const uint8_t* __restrict__ m, int lo, int hi, int32_t row_base,
                           int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int running = 0;
  for (int base = lo; base < hi; base += 64 * 16) {
    const int p0 = base + lane * 16;
    unsigned bits = p0 < hi ? mask_bits16(m, p0, hi) : 0u;
    const int c = __popc(bits);
    int pre = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) pre += __popcll(__ballot((c >> b) & 1) & below) << b;
    const int total = __shfl(pre + c, 63);
    int o = running + pre;
    while (bits) {
      const int j = __ffs(bits) - 1;
      bits &= bits - 1;
      out[o++] = row_base + p0 + j;
    }
    running += total;
  }
}

__global__ __launch_bounds__(kThreads) void k_mask_compact(const uint8_t* __restrict__ mask,
                                                           int64_t win_lo, int64_t win_hi,
                                                           int64_t block, PlanParams plan,
                                                           int32_t* __restrict__ idx,
                                                           int32_t* __restrict__ ctr) {
  __shared__ int s_first;
  __shared__ unsigned long long s_best;
  __shared__ int s_wave_total[kThreads / 64];
  __shared__ int s_pos[kChunk];  // one chunk's positions, in order, for coalesced stores
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int lo = (int)win_lo, hi = (int)win_hi;

  if (block > 0) {
    // First masked position of the window (min over threads, chunk by chunk).
    if (tid == 0) s_first = hi;
    __syncthreads();
    for (int base = lo; base < hi; base += kChunk) {
      const int p0 = base + tid * kPerThread;
      const unsigned fb = p0 < hi ? mask_bits16(mask, p0, hi) : 0u;
      if (fb) atomicMin(&s_first, p0 + __ffs(fb) - 1);
      __syncthreads();
      const bool found = s_first < hi;
      __syncthreads();
      if (found) break;
    }
    const int first = s_first;
    if (first >= hi) {
      lo = hi;
    } else {
      const int b = (int)((first - lo) / block);
      const int64_t blo = (int64_t)lo + (int64_t)b * block;
      const int64_t bhi = blo + block < (int64_t)hi ? blo + block : (int64_t)hi;
      lo = (int)blo;
      hi = (int)bhi;
    }
  }

  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int running = 0;
  for (int base = lo; base < hi; base += kChunk) {
    const int p0 = base + tid * kPerThread;
    unsigned bits = p0 < hi ? mask_bits16(mask, p0, hi) : 0u;
    const int c = __popc(bits);
    int pre = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {
      const unsigned long long bal = __ballot((c >> b) & 1);
      pre += __popcll(bal & below) << b;
    }
    if (lane == 63) s_wave_total[wave] = pre + c;
    __syncthreads();
    int wave_off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      const int t = s_wave_total[w];
      wave_off += (w < wave) ? t : 0;
      total += t;
    }
    // Each lane's positions go to LDS at its prefix, then the chunk's list
    // leaves in consecutive 4-byte stores across the workgroup.
    int out = wave_off + pre;
    while (bits) {
      const int j = __ffs(bits) - 1;
      bits &= bits - 1;
      s_pos[out++] = p0 + j;
    }
    __syncthreads();
    for (int i = tid; i < total; i += kThreads) idx[running + i] = s_pos[i];
    running += total;
    __syncthreads();  // s_wave_total and s_pos are rewritten by the next chunk
  }
  const int M = running;
  int S, n_rt;
  choose_plan(M, plan, &s_best, S, n_rt);
  if (tid == 0) {
    ctr[0] = M;
    ctr[1] = lo;
    ctr[2] = hi;
    ctr[3] = S;
    ctr[4] = n_rt;
  }
}

// Batched step: sequence b (length L, rows b * L + p) gets its own window
// and block; one wave per sequence at a time.  Pass 1 narrows each window
// and counts its candidates, an exclusive prefix over the sequences gives
// each its first row, pass 2 writes the rows; the sequences' (first row, M,
// k) go to req for the selection, and the plan is made for the total M.
__global__ __launch_bounds__(kThreads) void k_mask_compact_batch(const uint8_t* __restrict__ mask, int B,
                                                                 int64_t L, SeqTable seqs, int64_t block,
                                                                 PlanParams plan, int32_t* __restrict__ idx,
                                                                 int32_t* __restrict__ ctr,
                                                                 int32_t* __restrict__ req) {
  __shared__ int s_lo[kBatchMax], s_hi[kBatchMax], s_M[kBatchMax], s_start[kBatchMax];
  __shared__ int s_total;
  __shared__ unsigned long long s_best;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int b = wave; b < B; b += kThreads / 64) {
    const uint8_t* m = mask + (size_t)b * (size_t)L;
    int lo = seqs.lo[b], hi = seqs.hi[b];
    if (block > 0) wave_block_window(m, block, lo, hi);
    const int c = wave_count(m, lo, hi);
    if (lane == 0) {
      s_lo[b] = lo;
      s_hi[b] = hi;
      s_M[b] = c;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int b = 0; b < B; ++b) {
      s_start[b] = acc;
      acc += s_M[b];
    }
    s_total = acc;
  }
  __syncthreads();
  for (int b = wave; b < B; b += kThreads / 64) {
    wave_write(mask + (size_t)b * (size_t)L, s_lo[b], s_hi[b], (int32_t)((int64_t)b * L), idx + s_start[b]);
    if (lane == 0) {
      req[4 * b + 0] = s_start[b];
      req[4 * b + 1] = s_M[b];
      req[4 * b + 2] = seqs.k[b];
      req[4 * b + 3] = 0;
    }
  }
  const int M = s_total;
  int S, n_rt;
  choose_plan(M, plan, &s_best, S, n_rt);
  if (tid == 0) {
    ctr[0] = M;
    ctr[1] = 0;
    ctr[2] = 0;
    ctr[3] = S;
    ctr[4] = n_rt;
    ctr[5] = 0;
  }
}

// Small candidate windows (the host knows at most kSmallBM rows can come
// out): one wave, no barriers (find_few_rows).
__global__ __launch_bounds__(64) void k_mask_compact_small(const uint8_t* __restrict__ mask, int64_t win_lo,
                                                          int64_t win_hi, int64_t block, int fixed_slices,
                                                          int32_t* __restrict__ idx, int32_t* __restrict__ ctr) {
  const int lane = threadIdx.x;
  const FewRows f = find_few_rows(mask, win_lo, win_hi, block);
  if (f.cand) idx[f.slot] = f.lo + lane;
  if (lane == 0) {
    ctr[0] = f.M;
    ctr[1] = f.lo;
    ctr[2] = f.hi;
    ctr[3] = fixed_slices;
    ctr[4] = 1;
  }
}

}  // namespace

hipError_t launch_mask_compact_small(const uint8_t* mask, int64_t win_lo, int64_t win_hi, int64_t block,
                                     int fixed_slices, int32_t* idx, int32_t* ctr, hipStream_t stream) {
  hipLaunchKernelGGL(k_mask_compact_small, dim3(1), dim3(64), 0, stream, mask, win_lo, win_hi, block, fixed_slices,
                     idx, ctr);
  return hipGetLastError();
}

hipError_t launch_mask_compact_batch(const uint8_t* mask, int B, int64_t L, const SeqTable& seqs, int64_t block,
                                     PlanParams plan, int32_t* idx, int32_t* ctr, int32_t* req, hipStream_t stream) {
  hipLaunchKernelGGL(k_mask_compact_batch, dim3(1), dim3(kThreads), 0, stream, mask, B, L, seqs, block, plan, idx,
                     ctr, req);
  return hipGetLastError();
}

hipError_t launch_mask_compact(const uint8_t* mask, int64_t win_lo, int64_t win_hi, int64_t block,
                               PlanParams plan, int32_t* idx, int32_t* ctr, hipStream_t stream) {
  hipLaunchKernelGGL(k_mask_compact, dim3(1), dim3(kThreads), 0, stream, mask, win_lo, win_hi, block, plan,
                     idx, ctr);
  return hipGetLastError();
}

}  // namespace dllm
