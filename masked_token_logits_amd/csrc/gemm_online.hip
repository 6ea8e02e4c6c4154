// Masked LM-head GEMM with a fused online vocabulary reduction.
//
// For each candidate row r (hidden state of a masked position, gathered
// through the compacted index list) and each vocabulary entry v the logit is
// z[r][v] = sum_k hidden[idx[r]][k] * W_lm[v][k]  (Mosaic, Abstract: the
// LM-head logits computed only for masked positions).  The logits never
// leave registers: every workgroup owns one tile of rows and one slice of
// the vocabulary, walks the slice tile by tile in increasing vocabulary
// order and keeps, per row, the running maximum m, the lowest index a that
// attains it and s = sum exp(z - m) (the streaming form of max and
// log-sum-exp), rescaling s whenever m grows; with the extended statistics
// also the second-largest logit and sum exp(z - m) (z - m) for the margin
// and entropy scores (online_state.h).  One partial per (row, slice) is
// written; the merge kernel combines the slices.
//
// MI355X mapping
//   * bf16 MFMA v_mfma_f32_32x32x16_bf16: A operand = 32 vocabulary rows of
//     W_lm, B operand = 32 gathered hidden rows, fp32 accumulate.  With this
//     orientation each lane's 16 accumulators of a 32x32 block are 16
//     vocabulary entries of ONE row, so most of the reduction is in-lane.
//   * W_lm and hidden tiles are staged through LDS (BK = 64 bf16 per stage,
//     double buffered).  The few-row tile, which streams W_lm, keeps two
//     stages of global loads in flight in registers; the many-row tile one.
//     16-byte chunks are XOR-swizzled by row so that the ds_read_b128
//     fragment loads are bank-conflict free.
//   * The gather is fused: each thread resolves its hidden-row pointers
//     once through idx[] and streams them; no [M, d] copy exists.
//   * Workgroup ids are remapped so that the workgroups resident on one XCD
//     (ids congruent mod 8) own neighbouring (row tile, slice) pairs and
//     share hidden tiles in that XCD's L2.
//   * M is read on the device; row tiles past M exit at once, so the host
//     never waits for the compaction result.  For a single sequence the
//     few-row tile does the compaction itself: its candidate window holds at
//     most 32 positions, which one wave lists while the first W_lm loads are
//     in flight, so that step needs no compaction launch.
#include "readout_internal.h"

#include <math.h>

#include "few_rows.h"
#include "online_state.h"

namespace dllm {
namespace {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  constexpr int kXcd = 8;
  const int per = grid / kXcd, rem = grid % kXcd;
  const int x = bid % kXcd, loc = bid / kXcd;
  return (x < rem) ? x * (per + 1) + loc : rem * (per + 1) + (x - rem) * per + loc;
}

template <int BM_, int BN_, int WM_, int WN_, bool STREAM_W_ = false, int BK_ = kBK>
struct Tile {
  static constexpr bool STREAM_W = STREAM_W_;  // W_lm read exactly once: non-temporal loads
  // waves per SIMD to reserve registers for, from the workgroups the LDS
  // allows per CU (double-buffered W_lm and hidden stages): the streaming
  // tile's VGPRs must not be what limits its occupancy
  static constexpr int BK = BK_;              // K elements per LDS stage
  static constexpr int LDS_BYTES = 2 * (BN_ + BM_) * BK * 2;
  static constexpr int MIN_WAVES = STREAM_W ? (163840 / LDS_BYTES) * (WM_ * WN_) / 4 : 1;
  static constexpr int BM = BM_;             // candidate rows per workgroup
  static constexpr int BN = BN_;             // vocabulary entries per tile
  static constexpr int WM = WM_, WN = WN_;   // waves along rows / vocabulary
  static constexpr int NT = WM * WN * 64;
  static constexpr int WR = BM / WM;         // rows per wave
  static constexpr int WV = BN / WN;         // vocabulary entries per wave
  static constexpr int FR = WR / 32;         // 32x32 MFMA blocks along rows
  static constexpr int FV = WV / 32;         // along vocabulary
  static constexpr int CPR = BK / 8;         // 16-byte chunks per LDS row
  static constexpr int A_LD = BN * CPR / NT; // W chunks per thread per stage
  static constexpr int B_LD = BM * CPR / NT; // hidden chunks per thread per stage
  static_assert(BN * CPR % NT == 0 && BM * CPR % NT == 0, "tile / thread mismatch");
  static_assert(WR % 32 == 0 && WV % 32 == 0, "wave tile must be whole MFMA blocks");
  static_assert(CPR == 8 || CPR == 16, "swizzle: chunk ^ (row % CPR)");
};

// LDS element offset of 16-byte chunk `chunk` of row `row` in a [rows][CPR * 8]
// tile: chunks are XOR-swizzled by row so that the 16 consecutive rows of a
// ds_read_b128 phase hit distinct banks.
template <int CPR>
__device__ __forceinline__ int swz(int row, int chunk) { return row * (CPR * 8) + ((chunk ^ (row & (CPR - 1))) << 3); }

template <class T, bool EXT, bool FIND>
__global__ __launch_bounds__(T::NT, T::MIN_WAVES) void k_gemm_online(const uint16_t* __restrict__ W,
                                                       const uint16_t* __restrict__ H, int d, int V,
                                                       const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ ctr, int slices,
                                                       int n_vt, Partials part, FindRows fr) {
  static_assert(!FIND || (T::STREAM_W && T::BM == kSmallBM), "the row search is the few-row tile's");
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][T::BN * T::BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][T::BM * T::BK];

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = bid / slices;
  const int slice = bid - rt * slices;
  const int row0 = rt * T::BM;
  const int vt_lo = (int)(((int64_t)slice * n_vt) / slices);
  const int vt_hi = (int)(((int64_t)(slice + 1) * n_vt) / slices);
  int M = 0;
  if constexpr (!FIND) {
    M = ctr[0];
    if (row0 >= M || vt_lo >= vt_hi) return;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave / T::WN;  // wave row group
  const int wv = wave % T::WN;  // wave vocabulary group
  const int KT = (d + T::BK - 1) / T::BK;

  // Per-thread load assignments (fixed for the workgroup's life).
  int a_row[T::A_LD], a_ch[T::A_LD];
#pragma unroll
  for (int i = 0; i < T::A_LD; ++i) {
    const int c = i * T::NT + tid;
    a_row[i] = c / T::CPR;
    a_ch[i] = c % T::CPR;
  }
  const uint16_t* b_ptr[T::B_LD];
  int b_row[T::B_LD], b_ch[T::B_LD];
#pragma unroll
  for (int i = 0; i < T::B_LD; ++i) {
    const int c = i * T::NT + tid;
    b_row[i] = c / T::CPR;
    b_ch[i] = c % T::CPR;
  }
  // Hidden-row pointers through the candidate list (M > 0).
  auto set_rows = [&](const int32_t* list) {
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i) {
      int r = row0 + b_row[i];
      r = r < M ? r : M - 1;  // rows past M read a valid row; their results are dropped
      b_ptr[i] = H + (size_t)list[r] * (size_t)d;
    }
  };

  const bf16x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  // Global -> registers (one register set per stage in flight), registers ->
  // LDS.  The loads are unconditional: a chunk past d reads the row's last
  // chunk instead (d % 8 == 0, so that is in bounds) and is replaced by zeros
  // when stored, so no load sits in a branch and the compiler can leave a
  // later stage's loads in flight while an earlier stage is stored.
  // `spare`: a load past the workgroup's last stage, whose data is never
  // stored; it reads the thread's (L2-resident) first hidden row instead of
  // W_lm, so it costs no HBM traffic.
  auto gload_w = [&](int vt, int ks, bf16x8* ra, bool spare = false) {
    const int k0 = ks * T::BK;
    const int v0 = vt * T::BN;
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i) {
      int v = v0 + a_row[i];
      v = v < V ? v : V - 1;
      int k = k0 + a_ch[i] * 8;
      k = k < d ? k : d - 8;
      const uint16_t* row = spare ? b_ptr[0] : W + (size_t)v * (size_t)d;
      const bf16x8* src = reinterpret_cast<const bf16x8*>(row + k);
      if constexpr (T::STREAM_W)
        ra[i] = __builtin_nontemporal_load(src);
      else
        ra[i] = *src;
    }
  };
  auto gload_h = [&](int ks, bf16x8* rb) {
    const int k0 = ks * T::BK;
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i) {
      int k = k0 + b_ch[i] * 8;
      k = k < d ? k : d - 8;
      rb[i] = *reinterpret_cast<const bf16x8*>(b_ptr[i] + k);
    }
  };
  auto lstore = [&](int buf, int ks, const bf16x8* ra, const bf16x8* rb) {
    const int k0 = ks * T::BK;
#pragma unroll
    for (int i = 0; i < T::A_LD; ++i)
      *reinterpret_cast<bf16x8*>(&sA[buf][swz<T::CPR>(a_row[i], a_ch[i])]) = k0 + a_ch[i] * 8 < d ? ra[i] : zero8;
#pragma unroll
    for (int i = 0; i < T::B_LD; ++i)
      *reinterpret_cast<bf16x8*>(&sB[buf][swz<T::CPR>(b_row[i], b_ch[i])]) = k0 + b_ch[i] * 8 < d ? rb[i] : zero8;
  };

  f32x16 acc[T::FV][T::FR];
  RowState run[T::FR];
#pragma unroll
  for (int fr = 0; fr < T::FR; ++fr) run[fr] = row_state_empty();
#pragma unroll
  for (int fv = 0; fv < T::FV; ++fv)
#pragma unroll
    for (int fr = 0; fr < T::FR; ++fr)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[fv][fr][e] = 0.f;

  const int total = (vt_hi - vt_lo) * KT;
  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;

  // One stage: the MFMAs on LDS buffer `buf` (stage (vt, ks)), and after the
  // tile's last K stage the online reduction of the tile.
  auto body = [&](int buf, int vt, int ks) {
#pragma unroll
    for (int kk = 0; kk < T::BK / 16; ++kk) {
      const int ch = kk * 2 + frag_half;
      bf16x8 fa[T::FV], fb[T::FR];
#pragma unroll
      for (int fv = 0; fv < T::FV; ++fv) {
        const int r = wv * T::WV + fv * 32 + frag_row;
        fa[fv] = *reinterpret_cast<const bf16x8*>(&sA[buf][swz<T::CPR>(r, ch)]);
      }
#pragma unroll
      for (int fr = 0; fr < T::FR; ++fr) {
        const int r = wr * T::WR + fr * 32 + frag_row;
        fb[fr] = *reinterpret_cast<const bf16x8*>(&sB[buf][swz<T::CPR>(r, ch)]);
      }
#pragma unroll
      for (int fv = 0; fv < T::FV; ++fv)
#pragma unroll
        for (int fr = 0; fr < T::FR; ++fr)
          acc[fv][fr] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fv], fb[fr], acc[fv][fr], 0, 0, 0);
    }

    if (ks == KT - 1) {
      // Online reduction of this vocabulary tile.  Accumulator e of block
      // (fv, fr) in this lane is vocabulary entry
      //   v0 + fv*32 + 8*(e/4) + 4*(lane/32) + e%4
      // of row wr*WR + fr*32 + lane%32; for a fixed lane these increase
      // with (fv, e), the order row_fold needs to keep the lowest index.
      const int v0 = vt * T::BN + wv * T::WV + 4 * frag_half;
      const bool full = (vt + 1) * T::BN <= V;
      auto off = [](int i) { return (i >> 4) * 32 + 8 * ((i & 15) >> 2) + (i & 3); };
#pragma unroll
      for (int fr = 0; fr < T::FR; ++fr) {
        float z[T::FV * 16];
#pragma unroll
        for (int i = 0; i < T::FV * 16; ++i) z[i] = acc[i >> 4][fr][i & 15];
        if (!full) {
          // Last vocabulary tile only: entries past V drop out (the limit
          // passes through an empty asm, so the compares stay in this
          // uniform branch instead of running on every tile).
          int lim = V - v0;
          asm volatile("" : "+v"(lim));
#pragma unroll
          for (int i = 0; i < T::FV * 16; ++i) z[i] = off(i) >= lim ? -INFINITY : z[i];
        }
        row_fold<EXT, T::FV * 16>(run[fr], z, v0, off);
      }
#pragma unroll
      for (int fv = 0; fv < T::FV; ++fv)
#pragma unroll
        for (int fr = 0; fr < T::FR; ++fr)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[fv][fr][e] = 0.f;
    }
  };
  auto next = [&](int& vt, int& ks) {
    if (++ks == KT) {
      ks = 0;
      ++vt;
    }
  };

  if constexpr (T::STREAM_W) {
    // Few rows, W_lm streamed from HBM: two stages of global loads in flight
    // (register sets 0 and 1, by stage parity; the loop runs stages in pairs
    // so the sets are never indexed at run time).  Stage s loads stage s + 2,
    // computes stage s and stores stage s + 1 (loaded two stages earlier).
    // Every load and LDS store is unconditional, so no memory operation sits
    // in a branch and the loads in flight are the same on every path: past
    // the last stage the loads repeat the last stage (an L2 hit) and the
    // stores fill a buffer that is never read again.
    bf16x8 ra0[T::A_LD], rb0[T::B_LD], ra1[T::A_LD], rb1[T::B_LD];
    int vt = vt_lo, ks = 0;        // stage being computed
    int ld_vt = vt_lo, ld_ks = 0;  // stage being loaded
    bool spare = false;            // the loads are past the last stage
    auto ld_next = [&]() {
      if (ld_vt != vt_hi - 1 || ld_ks != KT - 1)
        next(ld_vt, ld_ks);
      else
        spare = true;
    };
    // The first two stages' W_lm loads go out before the rows are known.
    gload_w(ld_vt, ld_ks, ra0);
    const int ks0 = ld_ks;
    ld_next();
    gload_w(ld_vt, ld_ks, ra1);
    const int ks1 = ld_ks;
    ld_next();
    if constexpr (FIND) {
      // The step's candidate rows, found by wave 0 while those loads are in
      // flight (every workgroup finds the same list; workgroup 0 publishes it
      // for the finish kernel).  Staged in LDS buffer sB[1], not used before
      // the loop's first store, which follows two barriers.
      int* s_idx = reinterpret_cast<int*>(&sB[1][0]);
      if (wave == 0) {
        const FewRows f = find_few_rows(fr.mask, fr.win_lo, fr.win_hi, fr.block);
        if (f.cand) {
          s_idx[f.slot] = f.lo + lane;
          if (blockIdx.x == 0) fr.idx[f.slot] = f.lo + lane;
        }
        if (lane == 0) {
          s_idx[kSmallBM] = f.M;
          if (blockIdx.x == 0) {
            fr.ctr[0] = f.M;
            fr.ctr[1] = f.lo;
            fr.ctr[2] = f.hi;
            fr.ctr[3] = slices;
            fr.ctr[4] = 1;
            fr.ctr[5] = 0;
          }
        }
      }
      __syncthreads();
      M = s_idx[kSmallBM];
      if (row0 >= M || vt_lo >= vt_hi) return;
      set_rows(s_idx);
    } else {
      set_rows(idx);
    }
    gload_h(ks0, rb0);
    gload_h(ks1, rb1);
    lstore(0, ks0, ra0, rb0);
    __syncthreads();
    int s = 0;
    for (; s + 1 < total; s += 2) {
      gload_w(ld_vt, ld_ks, ra0, spare);  // stage s + 2
      gload_h(ld_ks, rb0);
      ld_next();
      int st_vt = vt, st_ks = ks;     // stage s + 1
      next(st_vt, st_ks);
      body(0, vt, ks);
      lstore(1, st_ks, ra1, rb1);
      __syncthreads();
      vt = st_vt;
      ks = st_ks;
      gload_w(ld_vt, ld_ks, ra1, spare);  // stage s + 3
      gload_h(ld_ks, rb1);
      ld_next();
      next(st_vt, st_ks);             // stage s + 2
      body(1, vt, ks);
      lstore(0, st_ks, ra0, rb0);
      __syncthreads();
      vt = st_vt;
      ks = st_ks;
    }
    if (s < total) {  // odd stage count: the last stage is in buffer 0
      body(0, vt, ks);
      __syncthreads();
    }
  } else {
    // One stage of global loads in flight (registers), double-buffered LDS.
    set_rows(idx);
    bf16x8 ra[T::A_LD], rb[T::B_LD];
    int vt = vt_lo, ks = 0;
    gload_w(vt, ks, ra);
    gload_h(ks, rb);
    lstore(0, ks, ra, rb);
    __syncthreads();
    for (int s = 0; s < total; ++s) {
      int nvt = vt, nks = ks;
      next(nvt, nks);
      const bool has_next = (s + 1) < total;
      if (has_next) {
        gload_w(nvt, nks, ra);
        gload_h(nks, rb);
      }
      body(s & 1, vt, ks);
      if (has_next) lstore((s & 1) ^ 1, nks, ra, rb);
      __syncthreads();
      vt = nvt;
      ks = nks;
    }
  }

  // Combine the two half-waves (same rows, interleaved vocabulary entries).
#pragma unroll
  for (int fr = 0; fr < T::FR; ++fr) row_merge<EXT>(run[fr], shfl_xor_state(run[fr], 32));

  // Combine the WN waves that share rows, in wave order, through LDS.
  float* xm = reinterpret_cast<float*>(&sA[0][0]);
  int* xa = reinterpret_cast<int*>(xm + T::WN * T::BM);
  float* xs = reinterpret_cast<float*>(xa + T::WN * T::BM);
  float* xm2 = xs + T::WN * T::BM;
  float* xt = xm2 + T::WN * T::BM;
  static_assert(5 * T::WN * T::BM * 4 <= (int)sizeof(sA[0]), "LDS exchange area too small");
  if (frag_half == 0) {
#pragma unroll
    for (int fr = 0; fr < T::FR; ++fr) {
      const int r = wr * T::WR + fr * 32 + frag_row;
      xm[wv * T::BM + r] = run[fr].m;
      xa[wv * T::BM + r] = run[fr].a;
      xs[wv * T::BM + r] = run[fr].s;
      if (EXT) {
        xm2[wv * T::BM + r] = run[fr].m2;
        xt[wv * T::BM + r] = run[fr].t;
      }
    }
  }
  __syncthreads();
  for (int r = tid; r < T::BM; r += T::NT) {
    RowState x;
    x.m = xm[r];
    x.a = xa[r];
    x.s = xs[r];
    x.m2 = EXT ? xm2[r] : -INFINITY;
    x.t = EXT ? xt[r] : 0.f;
#pragma unroll
    for (int w = 1; w < T::WN; ++w) {
      RowState y;
      y.m = xm[w * T::BM + r];
      y.a = xa[w * T::BM + r];
      y.s = xs[w * T::BM + r];
      y.m2 = EXT ? xm2[w * T::BM + r] : -INFINITY;
      y.t = EXT ? xt[w * T::BM + r] : 0.f;
      row_merge<EXT>(x, y);
    }
    const int row = row0 + r;
    if (row < M) {
      const size_t o = (size_t)row * (size_t)slices + (size_t)slice;
      if constexpr (T::STREAM_W) {
        // few rows: one 16-byte record (m, a, s, 0) per partial in part.m
        // (and (m2, t) in part.m2), so a merge issues one load per
        // partial and array
        float4 rec;
        rec.x = x.m;
        rec.y = __int_as_float(x.a);
        rec.z = x.s;
        rec.w = 0.f;
        reinterpret_cast<float4*>(part.m)[o] = rec;
        if (EXT) reinterpret_cast<float2*>(part.m2)[o] = make_float2(x.m2, x.t);
      } else {
        part.m[o] = x.m;
        part.a[o] = x.a;
        part.s[o] = x.s;
        if (EXT) {
          part.m2[o] = x.m2;
          part.t[o] = x.t;
        }
      }
    }
  }
}

using LargeTile = Tile<kLargeBM, kLargeBN, 2, 4>;
// Few rows: every W_lm byte is used by one workgroup only, so the tiles are
// streamed with non-temporal loads (no L2 / Infinity Cache allocation):
// measured 180 -> 162 us per step on the LLaDA-like head.
using SmallTile = Tile<kSmallBM, kSmallBN, 1, 4, true>;
static_assert(kSmallBM + 1 <= SmallTile::BM * SmallTile::BK / 2, "candidate list must fit in sB[1]");

}  // namespace

hipError_t launch_gemm_large(const uint16_t* W, const uint16_t* H, int d, int V, const int32_t* idx,
                             const int32_t* ctr, int n_row_tiles, int slices, Partials p, hipStream_t stream) {
  const int n_vt = (V + LargeTile::BN - 1) / LargeTile::BN;
  const int grid = n_row_tiles * slices;
  const FindRows none = {};
  if (p.ext)
    hipLaunchKernelGGL((k_gemm_online<LargeTile, true, false>), dim3(grid), dim3(LargeTile::NT), 0, stream, W, H, d,
                       V, idx, ctr, slices, n_vt, p, none);
  else
    hipLaunchKernelGGL((k_gemm_online<LargeTile, false, false>), dim3(grid), dim3(LargeTile::NT), 0, stream, W, H,
                       d, V, idx, ctr, slices, n_vt, p, none);
  return hipGetLastError();
}

hipError_t launch_gemm_small(const uint16_t* W, const uint16_t* H, int d, int V, const int32_t* idx,
                             const int32_t* ctr, int slices, Partials p, const FindRows* find, hipStream_t stream) {
  const int n_vt = (V + SmallTile::BN - 1) / SmallTile::BN;
  const FindRows fr = find ? *find : FindRows{};
  if (find) {
    if (p.ext)
      hipLaunchKernelGGL((k_gemm_online<SmallTile, true, true>), dim3(slices), dim3(SmallTile::NT), 0, stream, W, H,
                         d, V, idx, ctr, slices, n_vt, p, fr);
    else
      hipLaunchKernelGGL((k_gemm_online<SmallTile, false, true>), dim3(slices), dim3(SmallTile::NT), 0, stream, W,
                         H, d, V, idx, ctr, slices, n_vt, p, fr);
  } else {
    if (p.ext)
      hipLaunchKernelGGL((k_gemm_online<SmallTile, true, false>), dim3(slices), dim3(SmallTile::NT), 0, stream, W,
                         H, d, V, idx, ctr, slices, n_vt, p, fr);
    else
      hipLaunchKernelGGL((k_gemm_online<SmallTile, false, false>), dim3(slices), dim3(SmallTile::NT), 0, stream, W,
                         H, d, V, idx, ctr, slices, n_vt, p, fr);
  }
  return hipGetLastError();
}

}  // namespace dllm
