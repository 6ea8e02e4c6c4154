// Work order and waits of the persistent GEMM (gemm_persistent.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dllm {

__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  constexpr int kXcd = 8;
  const int per = grid / kXcd, rem = grid % kXcd;
  const int x = bid % kXcd, loc = bid / kXcd;
  return (x < rem) ? x * (per + 1) + loc : rem * (per + 1) + (x - rem) * per + loc;
}

// Work-item order.  Items are (row tile, vocabulary slice) pairs, taken in
// blocks of 32 row tiles x 8 slices; inside a block, sub-blocks of 4 row
// tiles x 8 slices with the row tile fastest.  With 256 workgroups, a round
// of the persistent grid is one block, and the 32 workgroups of each XCD
// (consecutive positions after xcd_remap) hold one 4 x 8 sub-block: in an
// XCD's L2 every hidden tile is shared by 8 workgroups and every W_lm tile
// by 4, and all 8 XCDs stream the same 8 W_lm slices at the same time, so
// each W_lm tile leaves HBM once per 32 row tiles.  Edge blocks shrink; the
// map is a bijection onto [0, n_rt) x [0, S).
constexpr int kGroupRows = 32, kGroupSlices = 8, kSubRows = 4;

__device__ __forceinline__ void item_coords(int e, int n_rt, int S, int& rt, int& slice) {
  const int g = e / (kGroupRows * S);
  const int e1 = e - g * kGroupRows * S;
  const int rb = min(kGroupRows, n_rt - g * kGroupRows);
  const int h = e1 / (rb * kGroupSlices);
  const int el = e1 - h * rb * kGroupSlices;
  const int cb = min(kGroupSlices, S - h * kGroupSlices);
  const int nsub = rb / kSubRows;
  int r, c;
  if (el < nsub * kSubRows * cb) {
    const int sg = el / (kSubRows * cb);
    const int rem = el - sg * kSubRows * cb;
    c = rem / kSubRows;
    r = sg * kSubRows + (rem - c * kSubRows);
  } else {
    const int rem = el - nsub * kSubRows * cb;
    const int rr = rb - nsub * kSubRows;
    c = rem / rr;
    r = nsub * kSubRows + (rem - c * rr);
  }
  rt = g * kGroupRows + r;
  slice = h * kGroupSlices + c;
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and all its LDS operations are done, then barrier the
// workgroup.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier (s_barrier alone is not a memory fence).
template <int N>
__device__ __forceinline__ void stage_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace dllm
