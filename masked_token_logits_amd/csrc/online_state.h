// Streaming (online) per-row state of the vocabulary reduction, shared by
// the GEMM epilogues and the merge kernels.
//
// Over the logits z_v of one row seen so far (vocabulary entries in
// increasing order within a stream), the state holds
//   m   the largest logit, a the lowest index attaining it,
//   s   sum_v 2^(g_v),  g_v = z_v log2(e) - sc(m),  sc(m) = fl(m log2(e)),
// and, for the extended statistics (margin and entropy confidence),
//   m2  the second-largest logit (equal to m when the maximum repeats),
//   t   ln(2) sum_v 2^(g_v) g_v.
// Exponentials use v_exp_f32 (base 2), so every sum is kept relative to the
// rounded base-2 exponent sc(m) of its own maximum rather than to m itself:
// rescaling between two maxima then multiplies by 2^(sc(m_old) - sc(m_new)),
// which is exactly 1 while the maximum does not change, so no rounding
// residual is compounded fold after fold.  With q = m log2(e) - sc(m) (the
// residual, taken once at the end):
//   conf    = 2^q / s                   (largest softmax probability)
//   lse     = m + (log2 s - q) ln 2     (natural log-sum-exp)
//   margin  = conf (1 - e^(m2 - m))     (largest minus second-largest probability)
//   entropy = ln s - t / s              (-sum p ln p; independent of the reference)
// These are the statistics of the confidence- and entropy-driven unmasking
// policies (Accelerating Masked Diffusion Large Language Models: A Survey of
// Efficient Inference Techniques, Main Findings).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace dllm {

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;

// sc(m) = fl(m * log2(e)), rounded once: never fused into a neighbouring
// add, so that equal maxima always give bit-equal references.
__device__ __forceinline__ float log2_ref(float m) {
#pragma clang fp contract(off)
  return m * kLog2eF;
}

struct RowState {
  float m, s, m2, t;
  int a;
};

__device__ __forceinline__ RowState row_state_empty() {
  RowState r;
  r.m = -INFINITY;
  r.s = 0.f;
  r.m2 = -INFINITY;
  r.t = 0.f;
  r.a = 0x7FFFFFFF;
  return r;
}

// Merge two states.  Equal maxima keep the lower index, so the result does
// not depend on the merge order; EXT also merges m2 and t.
template <bool EXT>
__device__ __forceinline__ void row_merge(RowState& x, const RowState& y) {
  const bool take_y = (y.m > x.m) || (y.m == x.m && y.a < x.a);
  const float mn = fmaxf(x.m, y.m);
  const float sn = log2_ref(mn);
  const float dx = log2_ref(x.m) - sn, dy = log2_ref(y.m) - sn;  // <= 0; -inf or NaN for an empty side
  const float cx = (x.m == -INFINITY) ? 0.f : (dx == 0.f ? 1.f : __builtin_amdgcn_exp2f(dx));
  const float cy = (y.m == -INFINITY) ? 0.f : (dy == 0.f ? 1.f : __builtin_amdgcn_exp2f(dy));
  if (EXT) {
    const float tx = (x.m == -INFINITY) ? 0.f : cx * fmaf(dx * kLn2F, x.s, x.t);
    const float ty = (y.m == -INFINITY) ? 0.f : cy * fmaf(dy * kLn2F, y.s, y.t);
    x.t = tx + ty;
    x.m2 = fmaxf(fminf(x.m, y.m), fmaxf(x.m2, y.m2));
  }
  x.s = x.s * cx + y.s * cy;
  // mask select: a '?:' between the two fields can become a load through a
  // selected address, which keeps the states out of registers
  const int sel = -(int)take_y;
  x.a = (y.a & sel) | (x.a & ~sel);
  x.m = mn;
}

// max(a, b, c) in one v_max3_f32.  Written out because fmaxf on values the
// compiler cannot prove quiet (accumulators read through inline asm) costs a
// canonicalising v_max_f32 x, x, x per input first; the logits here are
// never signalling NaNs.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Fold N logits z[0..N-1] into the state; z[i] is vocabulary entry
// v0 + off(i) with off increasing in i.  Entries outside the vocabulary must
// be -inf (they then add nothing).  The block's argmax is the lowest index
// among equal maxima: strict '>' comparisons in order (EXT), or the maximum
// first and then the lowest i holding it.
template <bool EXT, int N, class Off>
__device__ __forceinline__ void row_fold(RowState& r, const float* z, int v0, Off off) {
  static_assert(N >= 3, "max3 tree");
  float bm = -INFINITY, b2 = -INFINITY;
  int bi = 0;
  if constexpr (EXT) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      b2 = __builtin_amdgcn_fmed3f(bm, b2, z[i]);  // second largest of {bm, b2, z} (bm >= b2)
      bi = z[i] > bm ? off(i) : bi;
      bm = fmaxf(bm, z[i]);
    }
  } else {
    bm = max3f(z[0], z[1], z[2]);
#pragma unroll
    for (int i = 3; i < N; i += 2) bm = max3f(bm, z[i], z[i + 1 < N ? i + 1 : i]);
#pragma unroll
    for (int i = N - 1; i >= 0; --i) bi = z[i] == bm ? off(i) : bi;
  }
  const float mn = fmaxf(r.m, bm);
  if (mn == -INFINITY) return;
  const float sc = log2_ref(mn);
  float sum = 0.f, tt = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float g = fmaf(z[i], kLog2eF, -sc);  // z log2(e) - sc, one rounding
    const float e = __builtin_amdgcn_exp2f(g);
    sum += e;
    // e * g with g clamped: an entry of -inf gives 0 * -256 = 0, not NaN;
    // below -256 e is 0 anyway, so the clamp changes nothing else
    if (EXT) tt = fmaf(e, fmaxf(g, -256.f), tt);
  }
  const float d = log2_ref(r.m) - sc;  // exactly 0 while the maximum is unchanged
  const float c = (r.m == -INFINITY) ? 0.f : (d == 0.f ? 1.f : __builtin_amdgcn_exp2f(d));
  if (EXT) {
    const float old_t = (r.m == -INFINITY) ? 0.f : c * fmaf(d * kLn2F, r.s, r.t);
    r.t = fmaf(tt, kLn2F, old_t);
    r.m2 = fmaxf(fminf(r.m, bm), fmaxf(r.m2, b2));
  }
  r.s = r.s * c + sum;
  r.a = (bm > r.m) ? v0 + bi : r.a;
  r.m = mn;
}

// Final statistics of a merged state.
struct RowStats {
  float conf, lse, margin, entropy;
};

template <bool EXT>
__device__ __forceinline__ RowStats row_finish(const RowState& r) {
  RowStats o;
  const float q = fmaf(r.m, kLog2eF, -log2_ref(r.m));  // rounding residual of sc(m), |q| <= ulp/2
  const float log2_s = __builtin_amdgcn_logf(r.s);     // v_log_f32: base 2
  o.conf = __builtin_amdgcn_exp2f(q) / r.s;
  o.lse = fmaf(log2_s - q, kLn2F, r.m);
  if (EXT) {
    const float e2 = (r.m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((r.m2 - r.m) * kLog2eF);
    o.margin = (1.0f - e2) * o.conf;
    o.entropy = log2_s * kLn2F - r.t / r.s;
  } else {
    o.margin = 0.f;
    o.entropy = 0.f;
  }
  return o;
}

// Score -> 32-bit key that orders like the float (larger score, larger key).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Ranking score of a row under the step's policy (0 conf, 1 margin, 2 -entropy).
__device__ __forceinline__ float policy_score(const RowStats& st, int score_kind) {
  return score_kind == 1 ? st.margin : (score_kind == 2 ? -st.entropy : st.conf);
}

// The state held by lane (lane ^ off) of the wave.
__device__ __forceinline__ RowState shfl_xor_state(const RowState& r, int off) {
  RowState y;
  y.m = __shfl_xor(r.m, off);
  y.s = __shfl_xor(r.s, off);
  y.m2 = __shfl_xor(r.m2, off);
  y.t = __shfl_xor(r.t, off);
  y.a = __shfl_xor(r.a, off);
  return y;
}

}  // namespace dllm
