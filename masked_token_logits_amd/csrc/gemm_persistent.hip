// Persistent, compute-bound masked LM-head GEMM with the fused online
// vocabulary reduction (same arithmetic as the streaming GEMM in
// gemm_online.hip: per row the running max m, the lowest index a attaining
// it and s = sum exp(z - m) over the vocabulary in increasing order; Mosaic,
// Abstract: logits only for masked positions, never materialised).
//
// MI355X mapping
//   * One 256-thread workgroup per CU (grid = CU count), each of the 4 waves
//     owning a 128 (rows) x 128 (vocabulary) block of the 256 x 256 tile:
//     16 v_mfma_f32_32x32x16_bf16 per 16-deep K step, 256 fp32 accumulators
//     per lane.  A operand = W_lm rows, B operand = gathered hidden rows, so a
//     lane's accumulators of one 32x32 block are 16 vocabulary entries of a
//     single row and the max / argmax / sum-exp reduction is mostly in-lane.
//   * Operands reach LDS by direct global->LDS DMA (global_load_lds_dwordx4):
//     no VGPR staging.  BK = 32, a 4-deep ring of (W tile, hidden tile)
//     stages (128 KiB of the 160 KiB LDS): three stages are in flight while
//     one is consumed.  Waits are explicit (s_waitcnt vmcnt(N) + s_barrier)
//     so the compiler's conservative vmcnt(0) never drains the ring.
//   * 16-byte chunks are XOR-swizzled by row ((row >> 1) & 3) so that the
//     ds_read_b128 fragment loads are bank-conflict free; the swizzle is
//     applied by choosing each lane's global source chunk, since a DMA lane
//     always lands at LDS base + 16 * lane.
//   * The gather is fused: the hidden rows of a row tile are resolved once
//     through idx[] per work item.
//   * Work items are (row tile, vocabulary slice) pairs of the device-side
//     plan (ctr[3] = slices, ctr[4] = row tiles) written by the compaction
//     kernel once M is known.  Workgroup b takes items q(b), q(b) + G, ...,
//     with q(b) remapped so that the 32 workgroups of one XCD take 32
//     consecutive items (neighbouring slices of the same row tiles): they
//     share hidden tiles in their XCD's L2, and all XCDs walk the same W_lm
//     tiles at the same time (shared in the Infinity Cache).
#include "readout_internal.h"

#include <math.h>

namespace dllm {
namespace {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
#define LDS_AS __attribute__((address_space(3)))

constexpr int BM = kPersistBM, BN = kPersistBN, BK = kPersistBK, NST = kPersistStages;
constexpr int NT = 256;
constexpr int TILE = BM * BK;                 // elements of one operand tile per stage
constexpr int DMA_ROWS = 16;                  // rows written by one wave-wide DMA (64 x 16 B)
constexpr int DMA_PER_OPERAND = BM / DMA_ROWS / 4;  // per wave per stage: 4
constexpr int DMA_PER_STAGE = 2 * DMA_PER_OPERAND;  // per wave per stage: 8
constexpr float kLog2e = 1.4426950408889634f;
static_assert(BM == BN, "square tile assumed by the loader");
static_assert(BK == 32, "swizzle and DMA layout assume 4 chunks of 16 B per row");

__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  constexpr int kXcd = 8;
  const int per = grid / kXcd, rem = grid % kXcd;
  const int x = bid % kXcd, loc = bid / kXcd;
  return (x < rem) ? x * (per + 1) + loc : rem * (per + 1) + (x - rem) * per + loc;
}

__device__ __forceinline__ void merge_state(float& m, int& a, float& s, float m2, int a2, float s2) {
  const bool take2 = (m2 > m) || (m2 == m && a2 < a);
  const float mn = fmaxf(m, m2);
  const float e1 = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m - mn) * kLog2e);
  const float e2 = (m2 == -INFINITY) ? 0.f : s2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
  a = take2 ? a2 : a;
  m = mn;
  s = e1 + e2;
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

__global__ __launch_bounds__(NT, 1) void k_gemm_persistent(const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ H, int d, int V,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ ctr,
                                                          float* __restrict__ part_m,
                                                          int32_t* __restrict__ part_a,
                                                          float* __restrict__ part_s) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[NST][2][TILE];

  const int M = ctr[0];
  const int S = ctr[3];
  const int n_rt = ctr[4];
  const int n_items = n_rt * S;
  const int n_vt = (V + BN - 1) / BN;
  const int KT = d / BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1;   // rows [wr * 128, +128)
  const int wv = wave & 1;    // vocabulary [wv * 128, +128)

  // DMA lane geometry: lane -> row (lane / 4) of a 16-row block, LDS chunk
  // position lane % 4, global chunk = position ^ ((row >> 1) & 3).
  const int dma_row = lane >> 2;
  const int dma_chunk = (lane & 3) ^ ((lane >> 3) & 3);
  // Fragment geometry: lane -> row lane % 32 of a 32-row block, K half lane / 32.
  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  const int frag_swz = (lane >> 1) & 3;

  for (int e = xcd_remap(blockIdx.x, gridDim.x); e < n_items; e += gridDim.x) {
    const int rt = e / S;
    const int slice = e - rt * S;
    const int row0 = rt * BM;
    const int vt_lo = (int)(((int64_t)slice * n_vt) / S);
    const int vt_hi = (int)(((int64_t)(slice + 1) * n_vt) / S);
    const int total = (vt_hi - vt_lo) * KT;

    // Hidden-row sources of this lane's B DMAs (rows past M repeat row M-1).
    const uint16_t* hsrc[DMA_PER_OPERAND];
#pragma unroll
    for (int i = 0; i < DMA_PER_OPERAND; ++i) {
      int r = row0 + (wave + 4 * i) * DMA_ROWS + dma_row;
      r = r < M ? r : M - 1;
      hsrc[i] = H + (size_t)idx[r] * (size_t)d + dma_chunk * 8;
    }

    // Issue bookkeeping: the next stage to load is (iss_vt, iss_k0) into ring slot iss_slot.
    int issued = 0, iss_vt = vt_lo, iss_k0 = 0, iss_slot = 0;
    const uint16_t* wsrc[DMA_PER_OPERAND];
    auto set_w_rows = [&](int vt) {
#pragma unroll
      for (int i = 0; i < DMA_PER_OPERAND; ++i) {
        int v = vt * BN + (wave + 4 * i) * DMA_ROWS + dma_row;
        v = v < V ? v : V - 1;
        wsrc[i] = W + (size_t)v * (size_t)d + dma_chunk * 8;
      }
    };
    set_w_rows(iss_vt);
    auto issue_next = [&]() {
      uint16_t* sa = &lds[iss_slot][0][0] + wave * DMA_ROWS * BK;
      uint16_t* sb = &lds[iss_slot][1][0] + wave * DMA_ROWS * BK;
#pragma unroll
      for (int i = 0; i < DMA_PER_OPERAND; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(wsrc[i] + iss_k0),
                                         (LDS_AS void*)(sa + i * 4 * DMA_ROWS * BK), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < DMA_PER_OPERAND; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(hsrc[i] + iss_k0),
                                         (LDS_AS void*)(sb + i * 4 * DMA_ROWS * BK), 16, 0, 0);
      ++issued;
      iss_slot = (iss_slot + 1) & (NST - 1);
      iss_k0 += BK;
      if (iss_k0 == d) {
        iss_k0 = 0;
        ++iss_vt;
        if (iss_vt < vt_hi) set_w_rows(iss_vt);
      }
    };

    float run_m[4], run_s[4];
    int run_a[4];
#pragma unroll
    for (int fr = 0; fr < 4; ++fr) {
      run_m[fr] = -INFINITY;
      run_s[fr] = 0.f;
      run_a[fr] = 0;
    }

    // Prologue: stages 0 .. NST-2 in flight.
#pragma unroll
    for (int p = 0; p < NST - 1; ++p)
      if (issued < total) issue_next();

    int q = 0;
    for (int vt = vt_lo; vt < vt_hi; ++vt) {
      f32x16 acc[4][4];
#pragma unroll
      for (int fv = 0; fv < 4; ++fv)
#pragma unroll
        for (int fr = 0; fr < 4; ++fr)
#pragma unroll
          for (int x = 0; x < 16; ++x) acc[fv][fr][x] = 0.f;

      for (int ks = 0; ks < KT; ++ks, ++q) {
        const int ahead = issued - 1 - q;  // stages after q already in flight (0..2)
        if (ahead >= 2)
          stage_sync<2 * DMA_PER_STAGE>();
        else if (ahead == 1)
          stage_sync<DMA_PER_STAGE>();
        else
          stage_sync<0>();
        // Every wave has finished reading stage q-1: its slot takes the next stage.
        if (issued < total) issue_next();

        const uint16_t* sa = &lds[q & (NST - 1)][0][0];
        const uint16_t* sb = &lds[q & (NST - 1)][1][0];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          const int chunk = ((kk * 2 + frag_half) ^ frag_swz) * 8;
          bf16x8 fa[4], fb[4];
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            fa[f] = *reinterpret_cast<const bf16x8*>(sa + (wv * 128 + f * 32 + frag_row) * BK + chunk);
            fb[f] = *reinterpret_cast<const bf16x8*>(sb + (wr * 128 + f * 32 + frag_row) * BK + chunk);
          }
#pragma unroll
          for (int fv = 0; fv < 4; ++fv)
#pragma unroll
            for (int fr = 0; fr < 4; ++fr)
              acc[fv][fr] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fv], fb[fr], acc[fv][fr], 0, 0, 0);
        }
      }

      // Online reduction of the finished vocabulary tile.  Accumulator x of
      // block (fv, fr) is vocabulary entry v0 + fv*32 + 8*(x/4) + x%4 of row
      // wr*128 + fr*32 + lane%32, with v0 = tile base + wv*128 + 4*(lane/32);
      // for a fixed lane the index grows with (fv, x), so a strict '>' scan
      // keeps the lowest index among equal maxima.
      const int v0 = vt * BN + wv * 128 + 4 * frag_half;
      const bool full = (vt + 1) * BN <= V;
#pragma unroll
      for (int fr = 0; fr < 4; ++fr) {
        float tm = -INFINITY;
        int ta = 0;
#pragma unroll
        for (int fv = 0; fv < 4; ++fv)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int v = v0 + fv * 32 + 8 * (x >> 2) + (x & 3);
            const float z = (full || v < V) ? acc[fv][fr][x] : -INFINITY;
            ta = z > tm ? v : ta;
            tm = fmaxf(tm, z);
          }
        const float mn = fmaxf(run_m[fr], tm);
        const float sc = (mn == -INFINITY) ? 0.f : mn * kLog2e;
        float sum = 0.f;
#pragma unroll
        for (int fv = 0; fv < 4; ++fv)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int v = v0 + fv * 32 + 8 * (x >> 2) + (x & 3);
            const float z = (full || v < V) ? acc[fv][fr][x] : -INFINITY;
            sum += __builtin_amdgcn_exp2f(fmaf(z, kLog2e, -sc));
          }
        const float old = (run_m[fr] == -INFINITY) ? 0.f : run_s[fr] * __builtin_amdgcn_exp2f(run_m[fr] * kLog2e - sc);
        run_s[fr] = old + sum;
        run_a[fr] = (tm > run_m[fr]) ? ta : run_a[fr];
        run_m[fr] = mn;
      }
    }

    // Half-waves hold the same rows with interleaved vocabulary entries.
#pragma unroll
    for (int fr = 0; fr < 4; ++fr) {
      const float m2 = __shfl_xor(run_m[fr], 32);
      const int a2 = __shfl_xor(run_a[fr], 32);
      const float s2 = __shfl_xor(run_s[fr], 32);
      merge_state(run_m[fr], run_a[fr], run_s[fr], m2, a2, s2);
    }
    // The two vocabulary halves (wv = 0, 1) of each row meet in LDS.  All DMAs
    // have landed (the last stage waited for vmcnt(0)); barrier before reuse.
    stage_sync<0>();
    float* xm = reinterpret_cast<float*>(&lds[0][0][0]);
    int* xa = reinterpret_cast<int*>(xm + 2 * BM);
    float* xs = reinterpret_cast<float*>(xa + 2 * BM);
    if (frag_half == 0) {
#pragma unroll
      for (int fr = 0; fr < 4; ++fr) {
        const int r = wr * 128 + fr * 32 + frag_row;
        xm[wv * BM + r] = run_m[fr];
        xa[wv * BM + r] = run_a[fr];
        xs[wv * BM + r] = run_s[fr];
      }
    }
    stage_sync<0>();
    {
      const int r = tid;  // NT == BM: one row per thread
      float m = xm[r], s = xs[r];
      int a = xa[r];
      merge_state(m, a, s, xm[BM + r], xa[BM + r], xs[BM + r]);
      const int row = row0 + r;
      if (row < M) {
        const size_t o = (size_t)row * (size_t)S + (size_t)slice;
        part_m[o] = m;
        part_a[o] = a;
        part_s[o] = s;
      }
    }
    // The next item's prologue overwrites the exchange area and counts vmcnt
    // from zero: drain the stores and the LDS reads first.
    stage_sync<0>();
  }
}

static_assert(NT == BM, "one thread per row in the final merge");

}  // namespace

hipError_t launch_gemm_persistent(const uint16_t* W, const uint16_t* H, int d, int V, const int32_t* idx,
                                  const int32_t* ctr, int grid, float* pm, int32_t* pa, float* ps,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(k_gemm_persistent, dim3(grid), dim3(NT), 0, stream, W, H, d, V, idx, ctr, pm, pa, ps);
  return hipGetLastError();
}

}  // namespace dllm
