// Ceiling probe of the compute-bound readout GEMM: the instruction mix of its
// whole-line main loop (gemm_persistent.hip) with nothing else -- no gather,
// no vocabulary fold, no partials -- on operands taken from a caller buffer
// of random bf16 values, so the matrix pipes see a realistic bit-toggle rate
// (the sustained MFMA clock of this chip depends on it).
//
//   mode 0: only the MFMAs: 16 v_mfma_f32_32x32x16_bf16 per K step on
//           fragments loaded once from `src`;
//   mode 1: per 64-deep stage and wave, 64 MFMAs, 32 ds_read_b128 fragment
//           loads and 16 whole-line global_load_lds DMAs (8 rows x 128 B)
//           from an L2-resident 4 MiB region of `src` per XCD, one barrier
//           with vmcnt(8): the main loop's schedule (8 DMAs after every
//           other MFMA pair of K steps 0 and 1, 8 after every pair of K
//           step 3) and LDS layout.
// One 256-thread workgroup per compute unit, one wave per SIMD, as the GEMM.
#include "dllm_probe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kRowBytes = 8192;           // operand rows of 4096 bf16
constexpr int kRegionRows = 512;          // per XCD region: 512 rows, 4 MiB
constexpr int kSlots = 5, kSlotElems = 256 * 64;

template <int MODE>
__global__ __launch_bounds__(256, 1) void k_probe(const uint16_t* __restrict__ src, int stages,
                                                   float* __restrict__ sink, uint64_t* __restrict__ clocks) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kSlots * kSlotElems];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 1, wv = wave & 1;
  const int frag_row = lane & 31, frag_half = lane >> 5, frag_swz = (frag_row >> 1) & 7;
  const char* region = reinterpret_cast<const char*>(src) + (size_t)(blockIdx.x % 8) * kRegionRows * kRowBytes;
  // fragments from the random source (rows of this wave, first 64 columns)
  bf16x8 fa[2][4], fb[2][4];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      fa[c][f] = *reinterpret_cast<const bf16x8*>(region + (size_t)(wv * 128 + f * 32 + frag_row) * kRowBytes +
                                                   (c * 2 + frag_half) * 16);
      fb[c][f] = *reinterpret_cast<const bf16x8*>(region + (size_t)(256 + (wr + 2 * f) * 32 + frag_row) * kRowBytes +
                                                   (c * 2 + frag_half) * 16);
    }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[i][j][x] = 0.f;
  int k0 = 0, slot = 0;
  auto frag = [&](int kk, int i, bf16x8* a, bf16x8* b) {
    const int f = i >> 1;
    const int chunk = ((kk * 2 + frag_half) ^ frag_swz) * 8;
    const int hs = slot == kSlots - 1 ? 0 : slot + 1;
    if ((i & 1) == 0)
      a[f] = *reinterpret_cast<const bf16x8*>(lds + slot * kSlotElems + (wv * 128 + f * 32 + frag_row) * 64 + chunk);
    else
      b[f] = *reinterpret_cast<const bf16x8*>(lds + hs * kSlotElems + ((wr + 2 * f) * 32 + frag_row) * 64 + chunk);
  };
  auto dma = [&](int j) {
    const int l = (wave + 4 * j) * 8 + (lane >> 3);            // 0..255
    const int c = (lane & 7) ^ ((l >> 1) & 7);
    const char* p = region + (size_t)l * kRowBytes + k0 * 2 + c * 16;
    __builtin_amdgcn_global_load_lds((const void*)p, (LDS_AS void*)(lds + slot * kSlotElems + (wave + 4 * j) * 512),
                                     16, 0, 0);
  };
  // issue: 0 no DMAs, 1 one after every MFMA pair, 2 / 3 DMAs 0-3 / 4-7
  // after every other pair
  auto kstep = [&](int cur, int kk, int issue) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int fv = (2 * m + t) >> 2, fr = (2 * m + t) & 3;
        acc[fv][fr] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][fv], fb[cur][fr], acc[fv][fr], 0, 0, 0);
      }
      if (MODE == 1) {
        if (issue == 1) dma(m);
        if (issue >= 2 && (m & 1) == 0) dma((issue - 2) * 4 + (m >> 1));
        frag(kk, m, fa[cur ^ 1], fb[cur ^ 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (MODE == 1) {
    // fill the ring once so the fragments read random data from the start
#pragma unroll
    for (int j = 0; j < 8; ++j) dma(j);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
  }
  // shader clock and constant-rate wall clock around the loop (workgroup 0, wave 0)
  uint64_t c0 = 0, w0 = 0;
  if (clocks && blockIdx.x == 0 && threadIdx.x == 0) {
    c0 = clock64();
    w0 = wall_clock64();
  }
  for (int q = 0; q < stages; ++q) {
    kstep(0, 1, 2);
    kstep(1, 2, 3);
    kstep(0, 3, 0);
    if (MODE == 1) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (0 << 8));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    kstep(1, 0, 1);
    k0 = (k0 + 64) & 4095;
    slot = slot == kSlots - 1 ? 0 : slot + 1;
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (clocks && blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = clock64() - c0;
    clocks[1] = wall_clock64() - w0;
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[i][j][lane & 15];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

size_t dllm_probe_source_bytes(void) { return (size_t)8 * kRegionRows * kRowBytes; }

int64_t dllm_probe_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

dllm_status dllm_probe_gemm_mix(int32_t mode, const uint16_t* src, int32_t stages, float* sink, int32_t grid,
                                uint64_t* clocks, void* stream) {
  if (!src || !sink || stages < 1 || grid < 1 || (mode != 0 && mode != 1)) return DLLM_ERR_INVALID_ARG;
  if (((uintptr_t)src & 15u) != 0) return DLLM_ERR_UNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (mode == 0)
    hipLaunchKernelGGL(k_probe<0>, dim3(grid), dim3(256), 0, st, src, stages, sink, clocks);
  else
    hipLaunchKernelGGL(k_probe<1>, dim3(grid), dim3(256), 0, st, src, stages, sink, clocks);
  return hipGetLastError() == hipSuccess ? DLLM_OK : DLLM_ERR_HIP;
}

}  // extern "C"
