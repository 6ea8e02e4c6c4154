// Persistent, compute-bound masked LM-head GEMM with the fused online
// vocabulary reduction (same arithmetic as the streaming GEMM in
// gemm_online.hip: per row the running max m, the lowest index a attaining
// it and s = sum exp(z - m) over the vocabulary in increasing order, plus
// the margin / entropy terms when asked for (online_state.h); Mosaic,
// Abstract: logits only for masked positions, never materialised).
//
// MI355X mapping
//   * One 256-thread workgroup per CU (grid = CU count), each of the 4 waves
//     owning 128 rows (four interleaved 32-row blocks) x 128 vocabulary
//     entries of the 256 x 256 tile:
//     16 v_mfma_f32_32x32x16_bf16 per 16-deep K step, 256 fp32 accumulators
//     per lane.  A operand = W_lm rows, B operand = gathered hidden rows, so a
//     lane's accumulators of one 32x32 block are 16 vocabulary entries of a
//     single row and the max / argmax / sum-exp reduction is mostly in-lane.
//   * Operands reach LDS by direct global->LDS DMA (global_load_lds_dwordx4):
//     no VGPR staging.  With d % 64 == 0 (persistent_items_wl) a stage is
//     64 deep and every DMA reads whole 128-byte lines, in a ring of five
//     32 KiB operand slots (all 160 KiB of LDS); otherwise (d % 32 == 0,
//     persistent_items) 32-deep stages of half lines in a 4-deep ring of
//     (W tile, hidden tile) slots.  Waits are explicit (s_waitcnt vmcnt(N) +
//     s_barrier) so the compiler's conservative vmcnt(0) never drains the
//     ring, and each stage's barrier comes before its last K step, so the
//     next stage's first fragments load while that K step's MFMAs run.
//   * 16-byte chunks are XOR-swizzled by row so that the ds_read_b128
//     fragment loads are bank-conflict free; the swizzle is
//     applied by choosing each lane's global source chunk, since a DMA lane
//     always lands at LDS base + 16 * lane.
//   * The gather is fused: the hidden rows of a row tile are resolved once
//     through idx[] per work item.
//   * The same main loop serves the FFN's GEMMs (MODE = kEpiStore /
//     kEpiSwiGLU): rows are then contiguous, every item is exactly one
//     256 x 256 output tile, and the epilogue stores bf16 (for the gate/up
//     projection, SiLU(gate) * up of paired 32-row weight blocks).
//   * Work items are (row tile, vocabulary slice) pairs of the device-side
//     plan (ctr[3] = slices, ctr[4] = row tiles) written by the compaction
//     kernel once M is known.  Workgroup b takes items q(b), q(b) + G, ...,
//     with q(b) remapped so that the 32 workgroups of one XCD take 32
//     consecutive items, and items ordered (item_coords) so that those 32
//     form a 4 row-tile x 8 slice block and all XCDs share the same slices.
#include "readout_internal.h"

#include <math.h>

#include <type_traits>

#include "online_state.h"
#include "persistent_sched.h"

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
static_assert(BM == BN, "square tile assumed by the loader");
static_assert(BK == 32, "swizzle and DMA layout assume 4 chunks of 16 B per row");

// Round-to-nearest-even float -> bfloat16 bits (finite inputs), two per word.
__device__ __forceinline__ uint32_t bf16_pack2(float lo, float hi) {
  uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  a += 0x7FFFu + ((a >> 16) & 1u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (a >> 16) | (b & 0xFFFF0000u);
}

// SiLU(g) * u in fp32: g / (1 + 2^(-g log2 e)) * u.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g / (1.0f + __builtin_amdgcn_exp2f(-g * kLog2eF)) * u;
}

// MODE: kEpiReadout = online vocabulary reduction into per-slice partials
// (rows gathered through idx, M / slices / row tiles from ctr); kEpiStore /
// kEpiSwiGLU = bf16 output tiles (rows row 0..M-1 of H, shape from st).
// This is the main loop for d % 64 != 0 (d % 32 == 0): NST slots of (W_lm
// tile [256][32], hidden tile [256][32]), every DMA reading 64 bytes of each
// of 16 rows (half lines).  It keeps 32-bit source offsets, so the host
// takes it only while the hidden tensor spans < 4 GiB.
template <int MODE, bool EXT>
__device__ __forceinline__ void persistent_items(uint16_t* __restrict__ lds, const uint16_t* __restrict__ W,
                                                 const uint16_t* __restrict__ H, int d, int V,
                                                 const int32_t* __restrict__ idx,
                                                 const int32_t* __restrict__ ctr, Partials part, StoreArgs st) {
  auto wslot = [&](int s) { return lds + s * 2 * TILE; };
  auto hslot = [&](int s) { return lds + s * 2 * TILE + TILE; };

  const int n_vt = (V + BN - 1) / BN;
  const int M = MODE == kEpiReadout ? ctr[0] : st.M;
  const int S = MODE == kEpiReadout ? ctr[3] : n_vt;           // store modes: one output tile per item
  const int n_rt = MODE == kEpiReadout ? ctr[4] : (st.M + BM - 1) / BM;
  const int n_items = n_rt * S;
  const int KT = d / BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS DMA addresses stay scalar
  const int wr = wave >> 1;   // row half: local 32-row blocks wr, wr + 2, wr + 4, wr + 6
  const int wv = wave & 1;    // vocabulary [wv * 128, +128)

  // LDS layout of a [256][32] bf16 operand tile: row r holds its four 16-byte
  // chunks at positions chunk ^ f(r), f(r) = (r >> 2) & 3.  A ds_read_b128
  // phase serves 16 lanes = 16 consecutive rows of one chunk; rows r and r+4k
  // share a 64-byte bank quarter ((r & 3) * 64 of each 256 bytes) and f gives
  // them distinct 16-byte positions, so the 16 reads hit 64 distinct banks
  // (measured: no LDS bank conflicts).  DMA lane geometry: lane -> row
  // (lane / 4) of a 16-row block, LDS position lane % 4, global chunk =
  // position ^ f(row) = position ^ ((lane >> 4) & 3).
  const int dma_row = lane >> 2;
  const int dma_chunk = (lane & 3) ^ ((lane >> 4) & 3);
  // Fragment geometry: lane -> row lane % 32 of a 32-row block, K half lane / 32.
  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  const int frag_swz = (lane >> 2) & 3;  // f(row) for row = 32-aligned base + lane % 32

  for (int e = xcd_remap(blockIdx.x, gridDim.x); e < n_items; e += gridDim.x) {
    int rt, slice;
    item_coords(e, n_rt, S, rt, slice);
    const int row0 = rt * BM;
    // Rows of the tile.  Local row l is in 32-row block l / 32; wave half wr
    // computes local blocks wr, wr + 2, wr + 4, wr + 6, so a partial tile
    // splits its blocks evenly between the two halves.  Readout: the n_rt
    // tiles interleave the global 32-row blocks (tile rt holds blocks rt,
    // rt + n_rt, ...), so the candidate rows spread evenly over the tiles
    // (M = 288 is 5 + 4 blocks instead of 8 + 1).  Store modes: contiguous
    // tiles.  nb = local blocks holding rows.
    const int nblk = (M + 31) / 32;
    const int nb = MODE == kEpiReadout ? (rt < nblk ? min(8, (nblk - rt - 1) / n_rt + 1) : 0)
                                       : min(8, max(0, (M - row0 + 31) / 32));
    auto grow = [&](int l) {
      return MODE == kEpiReadout ? ((l >> 5) * n_rt + rt) * 32 + (l & 31) : row0 + l;
    };
    const int vt_lo = (int)(((int64_t)slice * n_vt) / S);
    const int vt_hi = (int)(((int64_t)(slice + 1) * n_vt) / S);

    // DMA sources as 32-bit byte offsets from uniform 64-bit bases (the host
    // only takes this path when W_lm and hidden each span < 4 GiB), so the
    // loads use scalar-base addressing and each costs one VGPR.
    // Hidden rows past M repeat row M-1.
    uint32_t hoff[DMA_PER_OPERAND];
#pragma unroll
    for (int i = 0; i < DMA_PER_OPERAND; ++i) {
      int r = grow((wave + 4 * i) * DMA_ROWS + dma_row);
      r = r < M ? r : M - 1;
      const uint32_t src = MODE == kEpiReadout ? (uint32_t)idx[r] : (uint32_t)r;
      hoff[i] = (src * (uint32_t)d + (uint32_t)(dma_chunk * 8)) * 2u;
    }
    // W_lm DMA j of this wave: rows (wave + 4 j) * 16 + lane / 4, 64 bytes,
    // with the hidden tiles' geometry.
    uint32_t woff[DMA_PER_OPERAND];
#pragma unroll
    for (int j = 0; j < DMA_PER_OPERAND; ++j)
      woff[j] = (uint32_t)(((wave + 4 * j) * DMA_ROWS + dma_row) * d + dma_chunk * 8) * 2u;
    const char* Hb = reinterpret_cast<const char*>(H);

    // Issue bookkeeping.  Stage positions are issued in order, position q
    // = (iss_vt, iss_k0), 8 DMAs per wave: the W_lm and hidden tiles into
    // ring slot iss_h.  Position q + 4 is issued during stage q, into the
    // slot stage q has finished with, also past the item's last stage: those
    // DMAs re-read the item's last W_lm tile (valid memory) and are never
    // consumed.  The stage body is then branch-free.  Waits: stage q + 1 must
    // have landed; the positions behind it (q + 2, q + 3) may stay in flight,
    // 16 DMAs.  The item's final vmcnt(0) drains the extra DMAs.  Rows past V
    // (last vocabulary tile only) re-read a chunk of row V - 1; the epilogue
    // drops their logits.
    int iss_vt = vt_lo, iss_k0 = 0, iss_h = 0;
    auto issue_h = [&](int j) {
      uint16_t* sb = hslot(iss_h) + (wave + 4 * j) * DMA_ROWS * BK;
      const char* Hk = Hb + (size_t)iss_k0 * 2u;
      __builtin_amdgcn_global_load_lds((const void*)(Hk + hoff[j]), (LDS_AS void*)sb, 16, 0, 0);
    };
    // W_lm DMA j of position (iss_vt, iss_k0).  Rows past V read the last
    // chunk of row V - 1 instead: one unsigned min against a tile-uniform
    // limit (on a full tile the tile's own last chunk, which changes nothing).
    auto issue_w = [&](int j) {
      const int vbase = (iss_vt < vt_hi ? iss_vt : vt_hi - 1) * BN;
      const char* Wb = reinterpret_cast<const char*>(W + (size_t)vbase * (size_t)d + iss_k0);
      const int rows_in = min(V - vbase, BN);
      const uint32_t wlim = (uint32_t)(((rows_in - 1) * d + (BK - 8)) * 2);
      uint16_t* sa = wslot(iss_h) + (wave + 4 * j) * DMA_ROWS * BK;
      __builtin_amdgcn_global_load_lds((const void*)(Wb + min(woff[j], wlim)), (LDS_AS void*)sa, 16, 0, 0);
    };
    auto advance_issue = [&]() {
      iss_h = (iss_h + 1) & (NST - 1);
      iss_k0 += BK;
      if (iss_k0 == d) {
        iss_k0 = 0;
        ++iss_vt;
      }
    };
    auto issue_pos = [&]() {
#pragma unroll
      for (int m = 0; m < DMA_PER_OPERAND; ++m) issue_w(m);
#pragma unroll
      for (int j = 0; j < DMA_PER_OPERAND; ++j) issue_h(j);
      advance_issue();
    };
    static_assert(DMA_PER_OPERAND == 4, "4 W_lm + 4 hidden DMAs per position");

    // Running state per row block, one array per field (an array of
    // RowState structs is not split into registers and lands in scratch).
    float run_m[4], run_s[4], run_m2[4], run_t[4];
    int run_a[4];
#pragma unroll
    for (int fr = 0; fr < 4; ++fr) {
      const RowState e0 = row_state_empty();
      run_m[fr] = e0.m;
      run_s[fr] = e0.s;
      run_m2[fr] = e0.m2;
      run_t[fr] = e0.t;
      run_a[fr] = e0.a;
    }
    auto get = [&](int fr) {
      RowState r;
      r.m = run_m[fr];
      r.s = run_s[fr];
      r.m2 = run_m2[fr];
      r.t = run_t[fr];
      r.a = run_a[fr];
      return r;
    };
    auto put = [&](int fr, const RowState& r) {
      run_m[fr] = r.m;
      run_s[fr] = r.s;
      run_m2[fr] = r.m2;
      run_t[fr] = r.t;
      run_a[fr] = r.a;
    };

    // Fragment loads of K step kk (0/1) of a stage: W_lm from slot ws,
    // hidden from slot hs.  Fragment i (i = 0..7) is W_lm block i/2 when i is
    // even, hidden block i/2 when odd, so the first MFMA's operands arrive
    // first.
    auto load_frag = [&](int ws, int hs, int kk, int i, bf16x8* fa, bf16x8* fb) {
      const int f = i >> 1;
      if ((i & 1) == 0) {
        const int chunk = ((kk * 2 + frag_half) ^ frag_swz) * 8;
        fa[f] = *reinterpret_cast<const bf16x8*>(wslot(ws) + (wv * 128 + f * 32 + frag_row) * BK + chunk);
      } else {
        const int chunk = ((kk * 2 + frag_half) ^ frag_swz) * 8;
        fb[f] = *reinterpret_cast<const bf16x8*>(hslot(hs) + ((wr + 2 * f) * 32 + frag_row) * BK + chunk);
      }
    };

    // The item's tiles for a wave whose NFR (0..4) first 32-row blocks
    // (local blocks wr, wr + 2, ...) hold rows (the rest of a partial row
    // tile is padding): MFMAs,
    // hidden fragment loads and the epilogue run for those blocks only,
    // while every wave issues the same DMAs and meets the same barriers.
    auto run_tiles = [&](auto nfr_tag) {
      constexpr int NFR = decltype(nfr_tag)::value;
      // Fragment i of a K step: W_lm block i/2 when i is even (needed while
      // any block is active), hidden block i/2 when odd (if that block is).
      auto frag = [&](int ws, int hs, int kk, int i, bf16x8* fa, bf16x8* fb) {
        if ((i & 1) == 0 ? NFR > 0 : (i >> 1) < NFR) load_frag(ws, hs, kk, i, fa, fb);
      };

      // Prologue: positions 0..2 in flight, wait for position 0, queue
      // position 3, fetch stage 0's first fragments.
      issue_pos();
      issue_pos();
      issue_pos();
      stage_sync<16>();  // position 0
      issue_pos();
      bf16x8 fxa[4], fxb[4], fya[4], fyb[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) frag(0, 0, 0, i, fxa, fxb);

      // One stage q: load the second K step's fragments while the first K
      // step's 16 MFMAs run; mid-stage barrier (stage q+1 landed, everyone is
      // done with stage q); queue stage q+4 into stage q's slot and load stage
      // q+1's first fragments while the second K step's 16 MFMAs run.  The
      // sched_barrier pattern spreads the fragment loads and DMAs between the
      // MFMAs, so the matrix pipe never waits on a burst of memory
      // instructions.  FIRST = first stage of a vocabulary tile: its first
      // MFMAs take an inline zero accumulator instead of acc, so acc is never
      // explicitly cleared (explicit clears get hoisted above the epilogue's
      // reads and force the accumulators out of AGPRs).
      f32x16 acc[4][4];
      const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      int cs = 0;  // stage q's ring slot
      auto stage = [&](auto first_tag) {
        constexpr bool FIRST = decltype(first_tag)::value;
        const int ns = (cs + 1) & (NST - 1);  // stage q + 1's slot
        // First K step: MFMA pair m (blocks 2m, 2m+1), then the second K
        // step's fragment m.  sched_barrier fixes the interleave.
#pragma unroll
        for (int m = 0; m < 8; ++m) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int fv = (2 * m + t) >> 2, fr = (2 * m + t) & 3;
            if (fr < NFR)
              acc[fv][fr] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fxa[fv], fxb[fr], FIRST ? zero16 : acc[fv][fr],
                                                                    0, 0, 0);
          }
          frag(cs, cs, 1, m, fya, fyb);
          __builtin_amdgcn_sched_barrier(0);
        }
        // Stage q+1 landed: positions q+2 and q+3 (8 + 8 DMAs) may stay in flight.
        stage_sync<16>();
        // Second K step: MFMA pair m, position q+4's DMAs (W_lm DMA m and
        // hidden DMA m for m < 4), fragment m of stage q+1's first K step.
#pragma unroll
        for (int m = 0; m < 8; ++m) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int fv = (2 * m + t) >> 2, fr = (2 * m + t) & 3;
            if (fr < NFR) acc[fv][fr] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fya[fv], fyb[fr], acc[fv][fr], 0, 0, 0);
          }
          if (m < 4)
            issue_w(m);
          else
            issue_h(m - 4);
          frag(ns, ns, 0, m, fxa, fxb);
          __builtin_amdgcn_sched_barrier(0);
        }
        advance_issue();
        cs = ns;
      };
      for (int vt = vt_lo; vt < vt_hi; ++vt) {
        stage(std::true_type{});
        for (int ks = 1; ks < KT; ++ks) stage(std::false_type{});
        if constexpr (NFR > 0) {
          // Online reduction of the finished vocabulary tile, one 16-value
          // block at a time.  Accumulator x of block (fv, fr) is vocabulary
          // entry v0 + fv*32 + 8*(x/4) + x%4 of local row (wr + 2 fr)*32 + lane%32,
          // with v0 = tile base + wv*128 + 4*(lane/32).  Within a lane the
          // index grows with (fv, x), the order row_fold needs to keep the
          // lowest index among equal maxima.
          // The accumulators are read with explicit v_accvgpr_read (inline
          // asm): left to itself the register allocator copies all 256 of
          // them to VGPRs at once and spills.  The compiler does not see these
          // reads as consumers of the MFMA results for hazard purposes, so 24
          // wait states are inserted first, ordered after every MFMA by
          // taking all live accumulators as operands.
          if constexpr (NFR == 4)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::"a"(acc[0][0]), "a"(acc[0][1]), "a"(acc[0][2]),
                         "a"(acc[0][3]), "a"(acc[1][0]), "a"(acc[1][1]), "a"(acc[1][2]), "a"(acc[1][3]),
                         "a"(acc[2][0]), "a"(acc[2][1]), "a"(acc[2][2]), "a"(acc[2][3]), "a"(acc[3][0]),
                         "a"(acc[3][1]), "a"(acc[3][2]), "a"(acc[3][3]));
          else if constexpr (NFR == 3)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::"a"(acc[0][0]), "a"(acc[0][1]), "a"(acc[0][2]),
                         "a"(acc[1][0]), "a"(acc[1][1]), "a"(acc[1][2]), "a"(acc[2][0]), "a"(acc[2][1]),
                         "a"(acc[2][2]), "a"(acc[3][0]), "a"(acc[3][1]), "a"(acc[3][2]));
          else if constexpr (NFR == 2)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::"a"(acc[0][0]), "a"(acc[0][1]), "a"(acc[1][0]),
                         "a"(acc[1][1]), "a"(acc[2][0]), "a"(acc[2][1]), "a"(acc[3][0]), "a"(acc[3][1]));
          else
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::"a"(acc[0][0]), "a"(acc[1][0]), "a"(acc[2][0]),
                         "a"(acc[3][0]));
          if constexpr (MODE == kEpiReadout) {
            const int v0 = vt * BN + wv * 128 + 4 * frag_half;
            const bool full = (vt + 1) * BN <= V;
            auto off = [](int x) { return 8 * (x >> 2) + (x & 3); };
#pragma unroll
            for (int fr = 0; fr < NFR; ++fr) {
#pragma unroll
              for (int fv = 0; fv < 4; ++fv) {
                float z[16];
#pragma unroll
                for (int x = 0; x < 16; ++x)
                  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(z[x]) : "a"(acc[fv][fr][x]));
                if (!full) {
                  // Last vocabulary tile only: entries past V drop out.  The
                  // limit passes through an empty asm so that neither the
                  // compares nor the selects move out of this (uniform)
                  // branch: there they would cost VALU on every tile.
                  int lim = V - (v0 + fv * 32);
                  asm volatile("" : "+v"(lim));
#pragma unroll
                  for (int x = 0; x < 16; ++x) z[x] = off(x) >= lim ? -INFINITY : z[x];
                }
                RowState r = get(fr);
                row_fold<EXT, 16>(r, z, v0 + fv * 32, off);
                put(fr, r);
              }
            }
          } else {
            // Output tile store (the item's only tile: these stores come after
            // the last stage's waits, and the item's vmcnt(0) drains them).
            // Accumulator x of block (fv, fr) is output column
            // c0 + fv*32 + 8*(x/4) + x%4, c0 = tile base + wv*128 + 4*(lane/32),
            // of row row0 + (wr + 2 fr)*32 + lane%32: four runs of 4 columns.
#pragma unroll
            for (int fr = 0; fr < NFR; ++fr) {
              const int row = row0 + (wr + 2 * fr) * 32 + frag_row;
              const bool ok = row < M;
              uint16_t* orow = st.out + (size_t)(ok ? row : 0) * (size_t)st.ldo;
              if constexpr (MODE == kEpiStore) {
                const int c0 = vt * BN + wv * 128 + 4 * frag_half;
#pragma unroll
                for (int fv = 0; fv < 4; ++fv) {
#pragma unroll
                  for (int j = 0; j < 4; ++j) {
                    float z[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                      asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(z[i]) : "a"(acc[fv][fr][4 * j + i]));
                    const uint2 pk = make_uint2(bf16_pack2(z[0], z[1]), bf16_pack2(z[2], z[3]));
                    if (ok) *reinterpret_cast<uint2*>(orow + c0 + fv * 32 + 8 * j) = pk;
                  }
                }
              } else {
                // Weight rows come in 64-row units: 32 gate rows, then the 32
                // up rows of the same outputs.  Blocks (0, 1) and (2, 3) of a
                // wave are such pairs, so gate and up of one output sit in the
                // same lane and register position.  Output column
                // c0 + p*32 + 8*(x/4) + x%4, c0 = tile*128 + wv*64 + 4*(lane/32).
                const int c0 = vt * (BN / 2) + wv * 64 + 4 * frag_half;
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
                  for (int j = 0; j < 4; ++j) {
                    float a[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                      float g, u;
                      asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(g) : "a"(acc[2 * pr][fr][4 * j + i]));
                      asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(u) : "a"(acc[2 * pr + 1][fr][4 * j + i]));
                      a[i] = swiglu(g, u);
                    }
                    const uint2 pk = make_uint2(bf16_pack2(a[0], a[1]), bf16_pack2(a[2], a[3]));
                    if (ok) *reinterpret_cast<uint2*>(orow + c0 + pr * 32 + 8 * j) = pk;
                  }
                }
              }
            }
          }
        }
      }
    };
    // this wave's blocks that hold rows: local blocks wr + 2 fr < nb
    const int nfr = min(4, max(0, (nb - wr + 1) / 2));
    switch (nfr) {
      case 4: run_tiles(std::integral_constant<int, 4>{}); break;
      case 3: run_tiles(std::integral_constant<int, 3>{}); break;
      case 2: run_tiles(std::integral_constant<int, 2>{}); break;
      case 1: run_tiles(std::integral_constant<int, 1>{}); break;
      default: run_tiles(std::integral_constant<int, 0>{}); break;
    }

    if constexpr (MODE == kEpiReadout) {
      // Half-waves hold the same rows with interleaved vocabulary entries.
  #pragma unroll
      for (int fr = 0; fr < 4; ++fr) {
        RowState x = get(fr), y;
        y.m = __shfl_xor(x.m, 32);
        y.s = __shfl_xor(x.s, 32);
        y.m2 = __shfl_xor(x.m2, 32);
        y.t = __shfl_xor(x.t, 32);
        y.a = __shfl_xor(x.a, 32);
        row_merge<EXT>(x, y);
        put(fr, x);
      }
      // The two vocabulary halves (wv = 0, 1) of each row meet in LDS.  All DMAs
      // have landed (the last stage waited for vmcnt(0)); barrier before reuse.
      stage_sync<0>();
      float* xm = reinterpret_cast<float*>(&lds[0]);
      int* xa = reinterpret_cast<int*>(xm + 2 * BM);
      float* xs = reinterpret_cast<float*>(xa + 2 * BM);
      float* xm2 = xs + 2 * BM;
      float* xt = xm2 + 2 * BM;
      if (frag_half == 0) {
  #pragma unroll
        for (int fr = 0; fr < 4; ++fr) {
          const int r = (wr + 2 * fr) * 32 + frag_row;
          xm[wv * BM + r] = run_m[fr];
          xa[wv * BM + r] = run_a[fr];
          xs[wv * BM + r] = run_s[fr];
          if (EXT) {
            xm2[wv * BM + r] = run_m2[fr];
            xt[wv * BM + r] = run_t[fr];
          }
        }
      }
      stage_sync<0>();
      {
        const int r = tid;  // NT == BM: one row per thread
        RowState x, y;
        x.m = xm[r];
        x.a = xa[r];
        x.s = xs[r];
        x.m2 = EXT ? xm2[r] : -INFINITY;
        x.t = EXT ? xt[r] : 0.f;
        y.m = xm[BM + r];
        y.a = xa[BM + r];
        y.s = xs[BM + r];
        y.m2 = EXT ? xm2[BM + r] : -INFINITY;
        y.t = EXT ? xt[BM + r] : 0.f;
        row_merge<EXT>(x, y);
        const int row = grow(r);  // >= M for local blocks past nb
        if (row < M) {
          const size_t o = (size_t)row * (size_t)S + (size_t)slice;
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
    // The next item's prologue overwrites the exchange area and counts vmcnt
    // from zero: drain the stores and the LDS reads first.
    stage_sync<0>();
  }
}

// Whole-line variant of the main loop (d % 64 == 0): 64-deep K stages, both
// operands streamed by DMAs that read whole 128-byte lines (8 rows x 128 B
// per wave instruction).  A stage is a hidden tile [256][64] and a W_lm tile
// [256][64], 32 KiB each, in a ring of NOP = 5 operand slots (160 KiB):
// operand i (the hidden tile of stage q is 2q, its W_lm tile 2q + 1) lives
// in slot i % 5.  Whole lines double what one CU can stream from L2 into LDS
// with four waves (measured 56 against 27.5 B/clk for 64-byte half lines).
//
// Stage q, four 16-deep K steps of 16 MFMAs per wave, each K step's MFMAs
// interleaved with the next K step's fragment loads:
//   K steps 0-1: also the DMAs of hidden tile q + 2 (into the slot W_lm tile
//                q - 1 held), after every other MFMA pair (one DMA per pair,
//                all in K step 0, measured 1-2% slower);
//   barrier B(q) after K step 2: this wave's reads of stage q are done
//                (lgkmcnt(0)) and stage q + 1 has landed (vmcnt(8): only
//                hidden tile q + 2 may be in flight);
//   K step 3:    also the DMAs of W_lm tile q + 2 (into the slot hidden tile
//                q held) and stage q + 1's first fragments.
// So hidden tiles are queued about two stages before use and W_lm tiles one
// (five slots allow no more; the other way round measured 7.5% slower on the
// 128k-position high-mask step, whose gathered hidden tiles stream from the
// Infinity Cache), and a wave meets one barrier per 64 MFMAs.
// The prologue queues the hidden and W_lm tiles of stages 0 and 1.
constexpr int WBK = kPersistWideBK;            // K per stage
constexpr int OPT = BM * WBK;                  // elements of one operand tile [256][64]
constexpr int NOP = 5;                         // operand slots
constexpr int WL_ROWS = 8;                     // rows per whole-line DMA
constexpr int WL_DMA = BM / WL_ROWS / 4;       // per wave, stage and operand: 8
static_assert(NOP * OPT * 2 <= 160 * 1024, "LDS budget of the whole-line ring");
static_assert(WL_DMA == 8, "the stage wait counts 8 DMAs per operand tile and wave");

template <int MODE, bool EXT>
__device__ __forceinline__ void persistent_items_wl(uint16_t* __restrict__ lds, const uint16_t* __restrict__ W,
                                                    const uint16_t* __restrict__ H, int d, int V,
                                                    const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ ctr, Partials part, StoreArgs st) {
  const int n_vt = (V + BN - 1) / BN;
  const int M = MODE == kEpiReadout ? ctr[0] : st.M;
  const int S = MODE == kEpiReadout ? ctr[3] : n_vt;           // store modes: one output tile per item
  const int n_rt = MODE == kEpiReadout ? ctr[4] : (st.M + BM - 1) / BM;
  const int n_items = n_rt * S;
  const int KT = d / WBK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS DMA addresses stay scalar
  const int wr = wave >> 1;   // row half: local 32-row blocks wr, wr + 2, wr + 4, wr + 6
  const int wv = wave & 1;    // vocabulary [wv * 128, +128)

  // LDS layout of a [256][64] bf16 operand tile: row r holds its eight
  // 16-byte chunks at positions chunk ^ fw(r), fw(r) = (r >> 1) & 7; the 16
  // rows of a ds_read_b128 phase then fill the 64 banks (even rows one half,
  // odd rows the other, 8 distinct positions each).  DMA lane geometry: lane
  // -> row lane / 8 of an 8-row block, LDS position lane % 8, global chunk
  // position ^ fw(row).
  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  const int frag_swz = (frag_row >> 1) & 7;

  for (int e = xcd_remap(blockIdx.x, gridDim.x); e < n_items; e += gridDim.x) {
    int rt, slice;
    item_coords(e, n_rt, S, rt, slice);
    const int row0 = rt * BM;
    const int nblk = (M + 31) / 32;
    const int nb = MODE == kEpiReadout ? (rt < nblk ? min(8, (nblk - rt - 1) / n_rt + 1) : 0)
                                       : min(8, max(0, (M - row0 + 31) / 32));
    auto grow = [&](int l) {
      return MODE == kEpiReadout ? ((l >> 5) * n_rt + rt) * 32 + (l & 31) : row0 + l;
    };
    const int vt_lo = (int)(((int64_t)slice * n_vt) / S);
    const int vt_hi = (int)(((int64_t)(slice + 1) * n_vt) / S);

    // DMA j (0..7) of this wave covers rows (wave + 4 j) * 8 + lane / 8 of
    // a tile; its lane reads global chunk (lane % 8) ^ fw(row).  Hidden rows
    // as 64-bit byte offsets (any hidden size), rows past M repeat row M - 1;
    // W_lm rows relative to the tile's first row.
    uint64_t hoff[WL_DMA];
    uint32_t woff[WL_DMA];
#pragma unroll
    for (int j = 0; j < WL_DMA; ++j) {
      const int l = (wave + 4 * j) * WL_ROWS + (lane >> 3);
      const int c = (lane & 7) ^ ((l >> 1) & 7);
      int r = grow(l);
      r = r < M ? r : M - 1;
      const uint64_t src = MODE == kEpiReadout ? (uint64_t)(uint32_t)idx[r] : (uint64_t)r;
      hoff[j] = (src * (uint64_t)d + (uint64_t)(c * 8)) * 2u;
      woff[j] = (uint32_t)((l * d + c * 8) * 2);
    }
    const char* Hb = reinterpret_cast<const char*>(H);

    // Issue bookkeeping: stage positions are numbered from the item's first
    // stage; the hidden tile of position q goes to slot (2q) % 5 and its
    // W_lm tile to (2q + 1) % 5.  Positions past the item's last stage
    // re-read its last W_lm tile and hidden tile (valid memory) and are never
    // consumed; the item's final vmcnt(0) drains them.  W_lm rows past V
    // (last vocabulary tile only) re-read a chunk of row V - 1; the epilogue
    // drops their logits.
    int wi_vt = vt_lo, wi_k0 = 0, wi_slot = 1;  // next W_lm position to issue
    int hi_k0 = 0, hi_slot = 0;                 // next hidden position to issue
    auto next_slot = [](int s) { return s + 2 >= NOP ? s + 2 - NOP : s + 2; };
    auto issue_w = [&](int j) {
      const int vbase = (wi_vt < vt_hi ? wi_vt : vt_hi - 1) * BN;
      const char* Wb = reinterpret_cast<const char*>(W + (size_t)vbase * (size_t)d + wi_k0);
      // Rows past V (last vocabulary tile only) read the last chunk of row
      // V - 1 instead: every valid row's offset is at most that chunk's, so
      // one unsigned min per DMA does it (on a full tile the limit is the
      // tile's own last chunk and changes nothing).
      const int rows_in = min(V - vbase, BN);
      const uint32_t wlim = (uint32_t)(((rows_in - 1) * d + (WBK - 8)) * 2);
      const uint32_t o = min(woff[j], wlim);
      __builtin_amdgcn_global_load_lds((const void*)(Wb + o),
                                       (LDS_AS void*)(lds + wi_slot * OPT + (wave + 4 * j) * WL_ROWS * WBK), 16, 0, 0);
    };
    auto advance_w = [&]() {
      wi_slot = next_slot(wi_slot);
      wi_k0 += WBK;
      if (wi_k0 == d) {
        wi_k0 = 0;
        ++wi_vt;
      }
    };
    auto issue_h = [&](int j) {
      const char* Hk = Hb + (size_t)hi_k0 * 2u;
      __builtin_amdgcn_global_load_lds((const void*)(Hk + hoff[j]),
                                       (LDS_AS void*)(lds + hi_slot * OPT + (wave + 4 * j) * WL_ROWS * WBK), 16, 0, 0);
    };
    auto advance_h = [&]() {
      hi_slot = next_slot(hi_slot);
      hi_k0 = hi_k0 + WBK == d ? 0 : hi_k0 + WBK;
    };

    float run_m[4], run_s[4], run_m2[4], run_t[4];
    int run_a[4];
#pragma unroll
    for (int fr = 0; fr < 4; ++fr) {
      const RowState e0 = row_state_empty();
      run_m[fr] = e0.m;
      run_s[fr] = e0.s;
      run_m2[fr] = e0.m2;
      run_t[fr] = e0.t;
      run_a[fr] = e0.a;
    }
    auto get = [&](int fr) {
      RowState r;
      r.m = run_m[fr];
      r.s = run_s[fr];
      r.m2 = run_m2[fr];
      r.t = run_t[fr];
      r.a = run_a[fr];
      return r;
    };
    auto put = [&](int fr, const RowState& r) {
      run_m[fr] = r.m;
      run_s[fr] = r.s;
      run_m2[fr] = r.m2;
      run_t[fr] = r.t;
      run_a[fr] = r.a;
    };

    auto run_tiles = [&](auto nfr_tag) {
      constexpr int NFR = decltype(nfr_tag)::value;
      // Fragment i (0..7) of K step kk of the stage in slots (ws, hs): W_lm
      // block i / 2 when i is even (needed while any block is active), hidden
      // block i / 2 when odd (if that block is).
      auto frag = [&](int ws, int hs, int kk, int i, bf16x8* fa, bf16x8* fb) {
        const int f = i >> 1;
        const int chunk = ((kk * 2 + frag_half) ^ frag_swz) * 8;
        if ((i & 1) == 0) {
          if (NFR > 0)
            fa[f] = *reinterpret_cast<const bf16x8*>(lds + ws * OPT + (wv * 128 + f * 32 + frag_row) * WBK + chunk);
        } else {
          if (f < NFR)
            fb[f] = *reinterpret_cast<const bf16x8*>(lds + hs * OPT + ((wr + 2 * f) * 32 + frag_row) * WBK + chunk);
        }
      };

      // Prologue: operands 0..3 (hidden and W_lm tiles of stages 0 and 1) in
      // flight; wait for stage 0 (stage 1 may stay: 16 DMAs); stage 0's first
      // fragments.
#pragma unroll
      for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int j = 0; j < WL_DMA; ++j) issue_h(j);
        advance_h();
#pragma unroll
        for (int j = 0; j < WL_DMA; ++j) issue_w(j);
        advance_w();
      }
      stage_sync<2 * WL_DMA>();
      bf16x8 fxa[4], fxb[4], fya[4], fyb[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) frag(1, 0, 0, i, fxa, fxb);

      f32x16 acc[4][4];
      const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      int cws = 1, chs = 0;  // stage q's W_lm and hidden slots
      // 16 MFMAs of one K step from fragments (a, b), in pairs, with
      // `between(m)` (m = 0..7: the memory work, here fragment m of the next
      // K step) after pair m.  Fragments load in the order W0, H0, W1, H1,
      // W2, H2, W3, H3, and the MFMAs run in the matching triangular order
      // (block (W k, H j) as soon as both are in): pair p of a K step uses
      // only fragments the previous K step loaded at least five pairs before
      // its end, so LDS latency never stalls the matrix pipe.  FIRST_K: the
      // first K step of a vocabulary tile takes an inline zero accumulator
      // (acc is never explicitly cleared: explicit clears get hoisted above
      // the epilogue's reads and push the accumulators out of AGPRs).
      auto kstep = [&](const bf16x8* a, const bf16x8* b, auto first_tag, auto between) {
        constexpr bool FIRST_K = decltype(first_tag)::value;
        // (W block, hidden block) of MFMA n
        constexpr int kOrder[16][2] = {{0, 0}, {1, 0}, {0, 1}, {1, 1}, {2, 0}, {2, 1}, {0, 2}, {1, 2},
                                       {2, 2}, {3, 0}, {3, 1}, {3, 2}, {0, 3}, {1, 3}, {2, 3}, {3, 3}};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int fv = kOrder[2 * m + t][0], fr = kOrder[2 * m + t][1];
            if (fr < NFR)
              acc[fv][fr] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fv], b[fr], FIRST_K ? zero16 : acc[fv][fr],
                                                                    0, 0, 0);
          }
          between(m);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      auto stage = [&](auto first_tag) {
        const int nws = next_slot(cws), nhs = next_slot(chs);  // stage q + 1's slots
        kstep(fxa, fxb, first_tag, [&](int m) {
          if ((m & 1) == 0) issue_h(m >> 1);
          frag(cws, chs, 1, m, fya, fyb);
        });
        kstep(fya, fyb, std::false_type{}, [&](int m) {
          if ((m & 1) == 0) issue_h(4 + (m >> 1));
          frag(cws, chs, 2, m, fxa, fxb);
        });
        advance_h();
        kstep(fxa, fxb, std::false_type{}, [&](int m) { frag(cws, chs, 3, m, fya, fyb); });
        // B(q): stage q + 1 landed (only the hidden tile of q + 2 may be in
        // flight) and every wave is done reading stage q.
        stage_sync<WL_DMA>();
        kstep(fya, fyb, std::false_type{}, [&](int m) {
          issue_w(m);
          frag(nws, nhs, 0, m, fxa, fxb);
        });
        advance_w();
        cws = nws;
        chs = nhs;
      };
      for (int vt = vt_lo; vt < vt_hi; ++vt) {
        stage(std::true_type{});
        for (int ks = 1; ks < KT; ++ks) stage(std::false_type{});
        if constexpr (NFR > 0) {
          // Online reduction of the finished vocabulary tile, one 16-value
          // block at a time.  Accumulator x of block (fv, fr) is vocabulary
          // entry v0 + fv*32 + 8*(x/4) + x%4 of local row (wr + 2 fr)*32 + lane%32,
          // with v0 = tile base + wv*128 + 4*(lane/32).  Within a lane the
          // index grows with (fv, x), the order row_fold needs to keep the
          // lowest index among equal maxima.
          // The accumulators are read with explicit v_accvgpr_read (inline
          // asm): left to itself the register allocator copies all 256 of
          // them to VGPRs at once and spills.  The compiler does not see these
          // reads as consumers of the MFMA results for hazard purposes, so 24
          // wait states are inserted first, ordered after every MFMA by
          // taking all live accumulators as operands.
          if constexpr (NFR == 4)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::"a"(acc[0][0]), "a"(acc[0][1]), "a"(acc[0][2]),
                         "a"(acc[0][3]), "a"(acc[1][0]), "a"(acc[1][1]), "a"(acc[1][2]), "a"(acc[1][3]),
                         "a"(acc[2][0]), "a"(acc[2][1]), "a"(acc[2][2]), "a"(acc[2][3]), "a"(acc[3][0]),
                         "a"(acc[3][1]), "a"(acc[3][2]), "a"(acc[3][3]));
          else if constexpr (NFR == 3)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::"a"(acc[0][0]), "a"(acc[0][1]), "a"(acc[0][2]),
                         "a"(acc[1][0]), "a"(acc[1][1]), "a"(acc[1][2]), "a"(acc[2][0]), "a"(acc[2][1]),
                         "a"(acc[2][2]), "a"(acc[3][0]), "a"(acc[3][1]), "a"(acc[3][2]));
          else if constexpr (NFR == 2)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::"a"(acc[0][0]), "a"(acc[0][1]), "a"(acc[1][0]),
                         "a"(acc[1][1]), "a"(acc[2][0]), "a"(acc[2][1]), "a"(acc[3][0]), "a"(acc[3][1]));
          else
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::"a"(acc[0][0]), "a"(acc[1][0]), "a"(acc[2][0]),
                         "a"(acc[3][0]));
          if constexpr (MODE == kEpiReadout) {
            const int v0 = vt * BN + wv * 128 + 4 * frag_half;
            const bool full = (vt + 1) * BN <= V;
            auto off = [](int x) { return 8 * (x >> 2) + (x & 3); };
#pragma unroll
            for (int fr = 0; fr < NFR; ++fr) {
#pragma unroll
              for (int fv = 0; fv < 4; ++fv) {
                float z[16];
#pragma unroll
                for (int x = 0; x < 16; ++x)
                  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(z[x]) : "a"(acc[fv][fr][x]));
                if (!full) {
                  // Last vocabulary tile only: entries past V drop out.  The
                  // limit passes through an empty asm so that neither the
                  // compares nor the selects move out of this (uniform)
                  // branch: there they would cost VALU on every tile.
                  int lim = V - (v0 + fv * 32);
                  asm volatile("" : "+v"(lim));
#pragma unroll
                  for (int x = 0; x < 16; ++x) z[x] = off(x) >= lim ? -INFINITY : z[x];
                }
                RowState r = get(fr);
                row_fold<EXT, 16>(r, z, v0 + fv * 32, off);
                put(fr, r);
              }
            }
          } else {
            // Output tile store (the item's only tile: these stores come after
            // the last stage's waits, and the item's vmcnt(0) drains them).
            // Accumulator x of block (fv, fr) is output column
            // c0 + fv*32 + 8*(x/4) + x%4, c0 = tile base + wv*128 + 4*(lane/32),
            // of row row0 + (wr + 2 fr)*32 + lane%32: four runs of 4 columns.
#pragma unroll
            for (int fr = 0; fr < NFR; ++fr) {
              const int row = row0 + (wr + 2 * fr) * 32 + frag_row;
              const bool ok = row < M;
              uint16_t* orow = st.out + (size_t)(ok ? row : 0) * (size_t)st.ldo;
              if constexpr (MODE == kEpiStore) {
                const int c0 = vt * BN + wv * 128 + 4 * frag_half;
#pragma unroll
                for (int fv = 0; fv < 4; ++fv) {
#pragma unroll
                  for (int j = 0; j < 4; ++j) {
                    float z[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                      asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(z[i]) : "a"(acc[fv][fr][4 * j + i]));
                    const uint2 pk = make_uint2(bf16_pack2(z[0], z[1]), bf16_pack2(z[2], z[3]));
                    if (ok) *reinterpret_cast<uint2*>(orow + c0 + fv * 32 + 8 * j) = pk;
                  }
                }
              } else {
                // Weight rows come in 64-row units: 32 gate rows, then the 32
                // up rows of the same outputs.  Blocks (0, 1) and (2, 3) of a
                // wave are such pairs, so gate and up of one output sit in the
                // same lane and register position.  Output column
                // c0 + p*32 + 8*(x/4) + x%4, c0 = tile*128 + wv*64 + 4*(lane/32).
                const int c0 = vt * (BN / 2) + wv * 64 + 4 * frag_half;
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
                  for (int j = 0; j < 4; ++j) {
                    float a[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                      float g, u;
                      asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(g) : "a"(acc[2 * pr][fr][4 * j + i]));
                      asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(u) : "a"(acc[2 * pr + 1][fr][4 * j + i]));
                      a[i] = swiglu(g, u);
                    }
                    const uint2 pk = make_uint2(bf16_pack2(a[0], a[1]), bf16_pack2(a[2], a[3]));
                    if (ok) *reinterpret_cast<uint2*>(orow + c0 + pr * 32 + 8 * j) = pk;
                  }
                }
              }
            }
          }
        }
      }
    };
    const int nfr = min(4, max(0, (nb - wr + 1) / 2));
    switch (nfr) {
      case 4: run_tiles(std::integral_constant<int, 4>{}); break;
      case 3: run_tiles(std::integral_constant<int, 3>{}); break;
      case 2: run_tiles(std::integral_constant<int, 2>{}); break;
      case 1: run_tiles(std::integral_constant<int, 1>{}); break;
      default: run_tiles(std::integral_constant<int, 0>{}); break;
    }
    if constexpr (MODE == kEpiReadout) {
      // Half-waves hold the same rows with interleaved vocabulary entries.
  #pragma unroll
      for (int fr = 0; fr < 4; ++fr) {
        RowState x = get(fr), y;
        y.m = __shfl_xor(x.m, 32);
        y.s = __shfl_xor(x.s, 32);
        y.m2 = __shfl_xor(x.m2, 32);
        y.t = __shfl_xor(x.t, 32);
        y.a = __shfl_xor(x.a, 32);
        row_merge<EXT>(x, y);
        put(fr, x);
      }
      // The two vocabulary halves (wv = 0, 1) of each row meet in LDS.  All DMAs
      // have landed (the last stage waited for vmcnt(0)); barrier before reuse.
      stage_sync<0>();
      float* xm = reinterpret_cast<float*>(&lds[0]);
      int* xa = reinterpret_cast<int*>(xm + 2 * BM);
      float* xs = reinterpret_cast<float*>(xa + 2 * BM);
      float* xm2 = xs + 2 * BM;
      float* xt = xm2 + 2 * BM;
      if (frag_half == 0) {
  #pragma unroll
        for (int fr = 0; fr < 4; ++fr) {
          const int r = (wr + 2 * fr) * 32 + frag_row;
          xm[wv * BM + r] = run_m[fr];
          xa[wv * BM + r] = run_a[fr];
          xs[wv * BM + r] = run_s[fr];
          if (EXT) {
            xm2[wv * BM + r] = run_m2[fr];
            xt[wv * BM + r] = run_t[fr];
          }
        }
      }
      stage_sync<0>();
      {
        const int r = tid;  // NT == BM: one row per thread
        RowState x, y;
        x.m = xm[r];
        x.a = xa[r];
        x.s = xs[r];
        x.m2 = EXT ? xm2[r] : -INFINITY;
        x.t = EXT ? xt[r] : 0.f;
        y.m = xm[BM + r];
        y.a = xa[BM + r];
        y.s = xs[BM + r];
        y.m2 = EXT ? xm2[BM + r] : -INFINITY;
        y.t = EXT ? xt[BM + r] : 0.f;
        row_merge<EXT>(x, y);
        const int row = grow(r);  // >= M for local blocks past nb
        if (row < M) {
          const size_t o = (size_t)row * (size_t)S + (size_t)slice;
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
    // The next item's prologue overwrites the exchange area and counts vmcnt
    // from zero: drain the stores and the LDS reads first.
    stage_sync<0>();
  }
}

static_assert(NT == BM, "one thread per row in the final merge");

template <int MODE, bool EXT>
__global__ __launch_bounds__(NT, 1) void k_gemm_persistent(const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ H, int d, int V,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ ctr, Partials part,
                                                          StoreArgs st) {
  // One array for both layouts (separate arrays make the compiler drain
  // vmcnt at every fragment read).
  __shared__ __attribute__((aligned(1024))) uint16_t lds[NOP * OPT];
  static_assert(NST * 2 * TILE <= NOP * OPT, "LDS layouts");
  if ((d & (WBK - 1)) == 0) {
    persistent_items_wl<MODE, EXT>(lds, W, H, d, V, idx, ctr, part, st);
    return;
  }
  persistent_items<MODE, EXT>(lds, W, H, d, V, idx, ctr, part, st);
}

}  // namespace

hipError_t launch_gemm_persistent(const uint16_t* W, const uint16_t* H, int d, int V, const int32_t* idx,
                                  const int32_t* ctr, int grid, Partials p, hipStream_t stream) {
  const StoreArgs none = {nullptr, 0, 0};
  if (p.ext)
    hipLaunchKernelGGL((k_gemm_persistent<kEpiReadout, true>), dim3(grid), dim3(NT), 0, stream, W, H, d, V, idx, ctr, p,
                       none);
  else
    hipLaunchKernelGGL((k_gemm_persistent<kEpiReadout, false>), dim3(grid), dim3(NT), 0, stream, W, H, d, V, idx, ctr,
                       p, none);
  return hipGetLastError();
}

hipError_t launch_gemm_store(bool swiglu, const uint16_t* W, int n_w_rows, const uint16_t* X, int K, int M,
                             uint16_t* out, int ldo, int grid, hipStream_t stream) {
  const Partials none = {};
  const StoreArgs st = {out, ldo, M};
  if (swiglu)
    hipLaunchKernelGGL((k_gemm_persistent<kEpiSwiGLU, false>), dim3(grid), dim3(NT), 0, stream, W, X, K, n_w_rows,
                       nullptr, nullptr, none, st);
  else
    hipLaunchKernelGGL((k_gemm_persistent<kEpiStore, false>), dim3(grid), dim3(NT), 0, stream, W, X, K, n_w_rows,
                       nullptr, nullptr, none, st);
  return hipGetLastError();
}

}  // namespace dllm
