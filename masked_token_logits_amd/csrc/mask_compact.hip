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
// from a small LDS table.  M and the window actually used go to ctr[0..2]
// so no host synchronisation is needed before the next kernel.
//
// The same kernel then fixes how the GEMM splits the work, now that M is
// known: for the persistent GEMM it picks the vocabulary slice count S that
// minimises (rounds of the persistent grid) x (longest item), each thread
// scoring one candidate and an LDS atomicMin choosing (ties: fewer slices).
#include "readout_internal.h"

namespace dllm {
namespace {

constexpr int kThreads = 1024;
constexpr int kPerThread = 16;
constexpr int kChunk = kThreads * kPerThread;

__global__ __launch_bounds__(kThreads) void k_mask_compact(const uint8_t* __restrict__ mask,
                                                           int64_t win_lo, int64_t win_hi,
                                                           int64_t block, PlanParams plan,
                                                           int32_t* __restrict__ idx,
                                                           int32_t* __restrict__ ctr) {
  __shared__ int s_first;
  __shared__ unsigned long long s_best;
  __shared__ int s_wave_total[kThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int lo = (int)win_lo, hi = (int)win_hi;

  if (block > 0) {
    // First masked position of the window (min over threads, chunk by chunk).
    if (tid == 0) s_first = hi;
    __syncthreads();
    for (int base = lo; base < hi; base += kChunk) {
      int mine = hi;
      const int p0 = base + tid * kPerThread;
#pragma unroll
      for (int j = kPerThread - 1; j >= 0; --j) {
        const int p = p0 + j;
        if (p < hi && mask[p] != 0) mine = p;
      }
      if (mine < hi) atomicMin(&s_first, mine);
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
    unsigned bits = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int p = p0 + j;
      if (p < hi && mask[p] != 0) bits |= 1u << j;
    }
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
    int out = running + wave_off + pre;
    while (bits) {
      const int j = __ffs(bits) - 1;
      bits &= bits - 1;
      idx[out++] = p0 + j;
    }
    running += total;
    __syncthreads();  // s_wave_total is rewritten by the next chunk
  }
  const int M = running;
  const int n_rt = (M + plan.tile_rows - 1) / plan.tile_rows;
  int S = plan.fixed_slices;
  if (S <= 0) {
    if (tid == 0) s_best = ~0ull;
    __syncthreads();
    if (n_rt > 0) {
      for (int c = tid + 1; c <= plan.max_slices && c <= plan.n_vt; c += kThreads) {
        if ((int64_t)n_rt * plan.tile_rows * c > plan.part_cap) break;
        const int64_t items = (int64_t)n_rt * c;
        const int64_t rounds = (items + plan.grid - 1) / plan.grid;
        const int64_t len = (plan.n_vt + c - 1) / c;  // vocabulary tiles of the longest item
        const unsigned long long cost = (unsigned long long)(rounds * (4 * len + 1));
        atomicMin(&s_best, (cost << 20) | (unsigned long long)c);
      }
    }
    __syncthreads();
    S = (s_best == ~0ull) ? 1 : (int)(s_best & 0xFFFFF);
  }
  if (tid == 0) {
    ctr[0] = M;
    ctr[1] = lo;
    ctr[2] = hi;
    ctr[3] = S;
    ctr[4] = n_rt;
  }
}

// Small candidate windows (the host knows at most 32 rows can come out): one
// wave, no barriers.  Block search reads 16 bytes per lane per iteration;
// the candidate block (<= 32 positions) is compacted with one ballot.
__global__ __launch_bounds__(64) void k_mask_compact_small(const uint8_t* __restrict__ mask, int64_t win_lo,
                                                          int64_t win_hi, int64_t block, int fixed_slices,
                                                          int32_t* __restrict__ idx, int32_t* __restrict__ ctr) {
  const int lane = threadIdx.x;
  int lo = (int)win_lo, hi = (int)win_hi;
  if (block > 0) {
    int first = hi;
    for (int base = lo; base < hi; base += 64 * 16) {
      int mine = hi;
      const int p0 = base + lane * 16;
#pragma unroll
      for (int j = 15; j >= 0; --j) {
        const int p = p0 + j;
        if (p < hi && mask[p] != 0) mine = p;
      }
      // lowest position over the wave: lanes cover increasing positions
      const unsigned long long bal = __ballot(mine < hi);
      if (bal) {
        first = __shfl(mine, __ffsll((long long)bal) - 1);
        break;
      }
    }
    if (first >= hi) {
      lo = hi;
    } else {
      const int64_t blo = win_lo + (int64_t)((first - lo) / block) * block;
      const int64_t bhi = blo + block < (int64_t)hi ? blo + block : (int64_t)hi;
      lo = (int)blo;
      hi = (int)bhi;
    }
  }
  const bool cand = lane < hi - lo && mask[lo + lane] != 0;  // hi - lo <= 32 here
  const unsigned long long bal = __ballot(cand);
  if (cand) idx[__popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))))] = lo + lane;
  if (lane == 0) {
    ctr[0] = __popcll(bal);
    ctr[1] = lo;
    ctr[2] = hi;
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

hipError_t launch_mask_compact(const uint8_t* mask, int64_t win_lo, int64_t win_hi, int64_t block,
                               PlanParams plan, int32_t* idx, int32_t* ctr, hipStream_t stream) {
  hipLaunchKernelGGL(k_mask_compact, dim3(1), dim3(kThreads), 0, stream, mask, win_lo, win_hi, block, plan,
                     idx, ctr);
  return hipGetLastError();
}

}  // namespace dllm
