// Device code of the few-row step: at most kSmallBM candidate rows, the
// current block of semi-autoregressive decoding (Sparse-dLLM, Experiment
// "Memory": logits only for the current block).  The candidate search is
// shared by the one-wave compaction kernel and the few-row GEMM (which, for
// a single sequence, finds its rows itself); the selection and commit is
// the last step of the few-row finish kernel.
#pragma once

#include "online_state.h"
#include "readout_internal.h"

namespace dllm {

// Bits j = 0..15 set where position p0 + j < hi holds a mask flag
// (p0 >= the window start).  One 16-byte load when the 16 bytes are aligned
// and inside the window, else byte loads.
__device__ __forceinline__ unsigned mask_bits16(const uint8_t* __restrict__ m, int p0, int hi) {
  unsigned bits = 0;
  if (p0 + 16 <= hi && (((uintptr_t)(m + p0)) & 15u) == 0) {
    const uint4 v = *reinterpret_cast<const uint4*>(m + p0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int by = 0; by < 4; ++by) bits |= ((w[q] >> (8 * by)) & 0xFFu) ? (1u << (4 * q + by)) : 0u;
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) bits |= (p0 + j < hi && m[p0 + j] != 0) ? (1u << j) : 0u;
  }
  return bits;
}

// Candidates of a window known to hold at most kSmallBM of them.
struct FewRows {
  int lo, hi;  // the candidate window actually used
  int M;       // number of candidates
  bool cand;   // this lane's position lo + lane is one ...
  int slot;    // ... at this index of the ascending list
};

// Called by one whole wave (lane = threadIdx.x & 63), no barrier.  Block-wise
// (block > 0): the window is cut into blocks of `block` positions from
// win_lo and the first one that holds a mask flag is searched: the first
// 1024 positions with one 16-byte load per lane (where a semi-autoregressive
// window normally finds its current block), the rest 64 positions per lane
// per iteration (four loads in flight).  The block's masked positions are
// then listed in ascending order with one ballot (the host guarantees
// hi - lo <= kSmallBM here).
__device__ __forceinline__ FewRows find_few_rows(const uint8_t* __restrict__ mask, int64_t win_lo, int64_t win_hi,
                                                 int64_t block) {
  const int lane = threadIdx.x & 63;
  int lo = (int)win_lo, hi = (int)win_hi;
  if (block > 0) {
    int first = hi;
    {
      const int64_t p = (int64_t)lo + lane * 16;
      const unsigned fb = p < hi ? mask_bits16(mask, (int)p, hi) : 0u;
      const int mine = fb ? (int)p + __ffs(fb) - 1 : hi;
      // lowest position over the wave: lanes cover increasing positions
      const unsigned long long bal = __ballot(mine < hi);
      if (bal) first = __shfl(mine, __ffsll((long long)bal) - 1);
    }
    if (first >= hi) {
      for (int64_t base = (int64_t)lo + 64 * 16; base < hi; base += 64 * 64) {  // 64-bit: no overflow near 2^31
        unsigned fb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t p = base + lane * 64 + 16 * j;
          fb[j] = p < hi ? mask_bits16(mask, (int)p, hi) : 0u;
        }
        int mine = hi;  // lowest flagged position of this lane's 64
#pragma unroll
        for (int j = 3; j >= 0; --j)
          if (fb[j]) mine = (int)(base + lane * 64 + 16 * j) + __ffs(fb[j]) - 1;
        const unsigned long long bal = __ballot(mine < hi);
        if (bal) {
          first = __shfl(mine, __ffsll((long long)bal) - 1);
          break;
        }
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
  FewRows f;
  f.cand = lane < hi - lo && mask[lo + lane] != 0;
  const unsigned long long bal = __ballot(f.cand);
  f.slot = __popcll(bal & ((1ull << lane) - 1ull));
  f.M = __popcll(bal);
  f.lo = lo;
  f.hi = hi;
  return f;
}

// Per-row results of the finish, in LDS.
struct FewRowSmem {
  float conf[kSmallBM], lse[kSmallBM], score[kSmallBM], margin[kSmallBM], ent[kSmallBM];
  int tok[kSmallBM], seq[kSmallBM];
  int n[kBatchMax];
};

// Selection + commit of at most kSmallBM rows whose results are in `sm`
// (every thread of the workgroup calls this; blockDim.x >= kSmallBM and
// >= the number of sequences).  Each row is ranked among the rows of its
// sequence by counting: row r precedes r' iff its score is larger, or equal
// with the lower row (= the lower position).  Each sequence commits its
// first n rows: n = min(k, M), or with the threshold rule
// n = min(max(#{score >= tau}, 1), k, M).  A batched step (req != nullptr)
// has rows b * L + p and outputs per sequence at b * k_stride (selection)
// and b * L (rows).
template <bool EXT>
__device__ __forceinline__ void few_rows_commit(FewRowSmem& sm, int M, const int32_t* __restrict__ idx,
                                                const int32_t* __restrict__ req, int B, int64_t L, int k_stride,
                                                const Policy& pol, int k, uint8_t* __restrict__ mask,
                                                int32_t* __restrict__ tokens, const dllm_step_out& o) {
  __syncthreads();
  const int t = threadIdx.x;
  const int nseq = req ? B : 1;
  if (t < nseq) {
    const int Mb = req ? req[4 * t + 1] : M;
    const int kb = req ? req[4 * t + 2] : k;
    int n = kb < Mb ? kb : Mb;
    if (pol.use_threshold && n > 0) {
      int cnt = 0;
      for (int r2 = 0; r2 < M; ++r2) cnt += (sm.seq[r2] == t && sm.score[r2] >= pol.tau) ? 1 : 0;
      n = cnt < 1 ? 1 : (cnt < n ? cnt : n);
    }
    sm.n[t] = n;
    if (o.n_out) o.n_out[t] = n;
    if (o.m_out) o.m_out[t] = Mb;
  }
  __syncthreads();
  if (t < M) {
    const int sq = sm.seq[t];
    const float c = sm.score[t];
    int rank = 0;
    for (int r2 = 0; r2 < M; ++r2) {
      const float c2 = sm.score[r2];
      rank += (sm.seq[r2] == sq && (c2 > c || (c2 == c && r2 < t))) ? 1 : 0;
    }
    const int64_t pos_base = (int64_t)sq * L;  // 0 for a single sequence (sq == 0)
    const int start = req ? req[4 * sq] : 0;
    const size_t slot = req ? (size_t)pos_base + (size_t)(t - start) : (size_t)t;
    const int g = idx[t];
    const int pos = (int)(g - pos_base);
    const int tok = sm.tok[t];
    if (o.row_idx) o.row_idx[slot] = pos;
    if (o.row_tok) o.row_tok[slot] = tok;
    if (o.row_conf) o.row_conf[slot] = sm.conf[t];
    if (o.row_lse) o.row_lse[slot] = sm.lse[t];
    if (EXT && o.row_margin) o.row_margin[slot] = sm.margin[t];
    if (EXT && o.row_entropy) o.row_entropy[slot] = sm.ent[t];
    if (rank < sm.n[sq]) {
      tokens[g] = tok;
      mask[g] = 0;
      const size_t sb = (size_t)sq * (size_t)k_stride + (size_t)rank;
      if (o.sel_idx) o.sel_idx[sb] = pos;
      if (o.sel_tok) o.sel_tok[sb] = tok;
      if (o.sel_conf) o.sel_conf[sb] = sm.conf[t];
    }
  }
}

}  // namespace dllm
