// Host side of the readout C ABI: argument checks, workspace carving, choice
// of the GEMM variant and launch of the step's kernels (compaction, GEMM,
// merge / selection) on the handle's stream.
#include "dllm_readout.h"
#include "readout_internal.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

// DLLM_DEBUG builds check the host-side invariants of workspace carving and
// launch planning (sizes each kernel's grid and indexing rely on) and abort
// with a message when one fails; release builds compile the checks out.
#ifdef DLLM_DEBUG
#define DLLM_DCHECK(cond)                                                                     \
  do {                                                                                        \
    if (!(cond)) {                                                                            \
      fprintf(stderr, "dllm: internal check failed at %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      abort();                                                                                \
    }                                                                                         \
  } while (0)
#else
#define DLLM_DCHECK(cond) \
  do {                    \
  } while (0)
#endif

// Scratch of dllm_masked_readout_step_noalloc: one array per GPU, held until
// the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: kernels get the address hipGetSymbolAddress returns for
// the current device (kept per device in scratch_ptr), never the name.
static __device__ __align__(256) uint8_t scratch[DLLM_NOALLOC_SCRATCH_BYTES];

struct dllm_readout {
  const uint16_t* W;
  int64_t V, d, L_max;
  int32_t k_max;
  hipStream_t stream;
  int cus;
  int slices_override;
  bool log;
  hipEvent_t ev_before, ev_after;
  dllm::Workspace ws;
};

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t small_slice_count(int64_t V) {
  const int64_t n_vt = (V + dllm::kSmallBN - 1) / dllm::kSmallBN;
  return n_vt < dllm::kMaxSmallSlices ? n_vt : dllm::kMaxSmallSlices;
}

bool limits_ok(int64_t L_max, int64_t d, int64_t V, int32_t k_max) {
  return L_max > 0 && L_max < (int64_t)1 << 31 && d > 0 && d < (int64_t)1 << 24 && V > 0 &&
         V < (int64_t)1 << 31 && k_max >= 0 && k_max <= DLLM_K_MAX_LIMIT;
}

// Byte offsets of each workspace array; returns the total size.
size_t carve(int64_t L_max, int64_t V, uint8_t* base, dllm::Workspace* ws) {
  // whole 256-row tiles times the largest slice count, so any plan with S <= 64 fits
  const int64_t part_cap_large = (L_max + dllm::kLargeBM - 1) / dllm::kLargeBM * dllm::kLargeBM *
                                 dllm::kMaxLargeSlices;
  // the few-row path stores 16-byte (m, a, s, 0) records in part_m: 4 floats per partial
  // (and 8-byte (m2, t) records in part_m2)
  const int64_t part_cap_small = 4 * (int64_t)dllm::kSmallBM * small_slice_count(V);
  const int64_t part_cap = part_cap_large > part_cap_small ? part_cap_large : part_cap_small;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes);
    return base ? base + o : nullptr;
  };
  dllm::Workspace w;
  w.idx = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)L_max));
  w.ctr = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * 16));
  w.part_m = reinterpret_cast<float*>(take(sizeof(float) * (size_t)part_cap));
  w.part_a = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)part_cap));
  w.part_s = reinterpret_cast<float*>(take(sizeof(float) * (size_t)part_cap));
  w.part_m2 = reinterpret_cast<float*>(take(sizeof(float) * (size_t)part_cap));
  w.part_t = reinterpret_cast<float*>(take(sizeof(float) * (size_t)part_cap));
  w.row_tok = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)L_max));
  w.row_conf = reinterpret_cast<float*>(take(sizeof(float) * (size_t)L_max));
  w.row_lse = reinterpret_cast<float*>(take(sizeof(float) * (size_t)L_max));
  w.keys = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (size_t)L_max));
  w.row_margin = reinterpret_cast<float*>(take(sizeof(float) * (size_t)L_max));
  w.row_entropy = reinterpret_cast<float*>(take(sizeof(float) * (size_t)L_max));
  w.req = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * 4 * (size_t)dllm::kBatchMax));
  w.part_cap = part_cap;
  DLLM_DCHECK(off % kAlign == 0);
  DLLM_DCHECK(part_cap >= (L_max + dllm::kLargeBM - 1) / dllm::kLargeBM * dllm::kLargeBM * dllm::kMaxLargeSlices);
  DLLM_DCHECK(part_cap >= 4 * (int64_t)dllm::kSmallBM * small_slice_count(V));
  DLLM_DCHECK(!base || (reinterpret_cast<uint8_t*>(w.req) + sizeof(int32_t) * 4 * (size_t)dllm::kBatchMax <=
                        base + off));
  if (ws) *ws = w;
  return off;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Vocabulary slices for the compute-bound path: enough workgroups to fill
// the device several times over, every slice at least one vocabulary tile.
int choose_large_slices(int n_row_tiles, int64_t V, int cus) {
  const int64_t n_vt = (V + dllm::kLargeBN - 1) / dllm::kLargeBN;
  int64_t s = (4 * (int64_t)cus + n_row_tiles - 1) / n_row_tiles;
  if (s < 1) s = 1;
  if (s > dllm::kMaxLargeSlices) s = dllm::kMaxLargeSlices;
  if (s > n_vt) s = n_vt;
  return (int)s;
}

dllm_status parse_policy(const dllm_policy* policy, dllm::Policy* pol) {
  *pol = {DLLM_SCORE_CONF, 0, 0.f};
  if (!policy) return DLLM_OK;
  if (policy->score < DLLM_SCORE_CONF || policy->score > DLLM_SCORE_NEG_ENTROPY) return DLLM_ERR_INVALID_ARG;
  if (policy->use_threshold != 0 && policy->use_threshold != 1) return DLLM_ERR_INVALID_ARG;
  if (policy->tau != policy->tau) return DLLM_ERR_INVALID_ARG;  // NaN
  pol->score = policy->score;
  pol->use_threshold = policy->use_threshold;
  pol->tau = policy->tau + 0.f;  // -0 -> +0: the kernels compare order-preserving bit patterns
  return DLLM_OK;
}

// A failed HIP call of a step: DLLM_ERR_HIP, and with DLLM_LOG=1 the call
// and HIP's description of the error on stderr.
dllm_status hip_failed(const dllm_readout* h, const char* what, hipError_t e) {
  if (h->log) fprintf(stderr, "[dllm] %s failed: %s (%d)\n", what, hipGetErrorString(e), (int)e);
  return DLLM_ERR_HIP;
}

dllm_status ensure_device(dllm_readout* h) {
  if (h->cus > 0) return DLLM_OK;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_failed(h, "hipGetDevice", e);
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_failed(h, "hipDeviceGetAttribute", e);
  if (cus <= 0) return DLLM_ERR_HIP;
  h->cus = cus;
  return DLLM_OK;
}

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

dllm_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DLLM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DLLM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DLLM_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return DLLM_OK;
}

// One validated step, single sequence (seqs == nullptr: k, win_lo, win_hi)
// or batched (B sequences of length L, rows b * L + p).
struct StepArgs {
  const uint16_t* hidden;
  int64_t L;
  uint8_t* mask;
  int32_t* tokens;
  int64_t block;
  int k;
  int64_t win_lo, win_hi;
  const dllm::SeqTable* seqs;
  int B;
  int64_t rows_max;     // host bound on the candidate rows of the step
  int64_t hidden_rows;  // rows of the hidden tensor (L or B * L)
};

dllm_status run_step(dllm_readout* h, const StepArgs& a, const dllm::Policy& pol, const dllm_step_out& o) {
  const dllm_status ds = ensure_device(h);
  if (ds != DLLM_OK) return ds;
  const dllm::Workspace& w = h->ws;
  const bool batched = a.seqs != nullptr;
  // margin / entropy are needed for ranking or output: keep (m2, t) too
  const bool ext = pol.score != DLLM_SCORE_CONF || o.row_margin != nullptr || o.row_entropy != nullptr;
  const dllm::Partials parts = {w.part_m, w.part_a, w.part_s, w.part_m2, w.part_t, ext};
  const int64_t rows_max = a.rows_max;
  const int V = (int)h->V, d = (int)h->d;
  hipStream_t st = h->stream;

  // Choose the GEMM variant from the host-known bound on M; the slice count
  // of the persistent variant is fixed on the device once M is known.  The
  // persistent kernel addresses the rows of a W_lm tile with 32-bit byte
  // offsets (256 rows x d < 4 GiB).  Hidden rows: 64-bit offsets in its
  // whole-line main loop (d % 64 == 0), 32-bit in the half-line one
  // (d % 64 == 32), which therefore needs a hidden tensor under 4 GiB.
  enum { kSmall, kPersistent, kStreaming } path;
  const int64_t n_vt_large = (h->V + dllm::kLargeBN - 1) / dllm::kLargeBN;
  const bool w_tile32 = (int64_t)dllm::kPersistBN * h->d * 2 < ((int64_t)1 << 32);
  const bool hidden32 = a.hidden_rows * h->d * 2 < ((int64_t)1 << 32);
  const bool persistent_ok =
      h->d % dllm::kPersistBK == 0 && w_tile32 && (h->d % dllm::kPersistWideBK == 0 || hidden32);
  dllm::PlanParams plan = {};
  int n_rt = 0;
  if (rows_max <= dllm::kSmallBM) {
    path = kSmall;
    plan.fixed_slices = (int)small_slice_count(h->V);
    plan.tile_rows = dllm::kSmallBM;
  } else if (persistent_ok) {
    path = kPersistent;
    int so = h->slices_override;
    if (so > n_vt_large) so = (int)n_vt_large;
    plan.fixed_slices = so;
    plan.tile_rows = dllm::kPersistBM;
    plan.n_vt = (int)n_vt_large;
    plan.grid = h->cus;
    plan.max_slices = 1024;
    plan.part_cap = w.part_cap;
  } else {
    path = kStreaming;
    n_rt = (int)((rows_max + dllm::kLargeBM - 1) / dllm::kLargeBM);
    int sl = h->slices_override > 0 ? h->slices_override : choose_large_slices(n_rt, h->V, h->cus);
    if (sl > n_vt_large) sl = (int)n_vt_large;
    plan.fixed_slices = sl;
    plan.tile_rows = dllm::kLargeBM;
  }
  // every (row, slice) partial of the plan fits the carved partial arrays
  DLLM_DCHECK(rows_max <= h->L_max && a.hidden_rows <= h->L_max && a.B >= 1 && a.B <= dllm::kBatchMax);
  DLLM_DCHECK(path != kSmall || 4 * (int64_t)dllm::kSmallBM * plan.fixed_slices <= w.part_cap);
  DLLM_DCHECK(path != kStreaming || (int64_t)n_rt * dllm::kLargeBM * plan.fixed_slices <= w.part_cap);
  DLLM_DCHECK(path != kPersistent || (persistent_ok && plan.grid > 0));
  // A single-sequence few-row step has no compaction launch: the GEMM's
  // workgroups find the candidate rows themselves.
  const bool fused = path == kSmall && !batched && rows_max > 0;
  hipError_t ce = hipSuccess;
  if (batched)
    ce = dllm::launch_mask_compact_batch(a.mask, a.B, a.L, *a.seqs, a.block, plan, w.idx, w.ctr, w.req, st);
  else if (path == kSmall && !fused)
    ce = dllm::launch_mask_compact_small(a.mask, a.win_lo, a.win_hi, a.block, plan.fixed_slices, w.idx, w.ctr, st);
  else if (path != kSmall)
    ce = dllm::launch_mask_compact(a.mask, a.win_lo, a.win_hi, a.block, plan, w.idx, w.ctr, st);
  if (ce != hipSuccess) return hip_failed(h, "compaction launch", ce);

  const int32_t* req = batched ? w.req : nullptr;
  const int k_stride = h->k_max;
  if (rows_max > 0) {
    hipError_t e;
    if (h->ev_before) {
      const hipError_t er = hipEventRecord(h->ev_before, st);
      if (er != hipSuccess) return hip_failed(h, "hipEventRecord", er);
    }
    if (path == kSmall) {
      const dllm::FindRows fr = {a.mask, a.win_lo, a.win_hi, a.block, w.idx, w.ctr};
      e = dllm::launch_gemm_small(h->W, a.hidden, d, V, w.idx, w.ctr, plan.fixed_slices, parts,
                                  fused ? &fr : nullptr, st);
    } else if (path == kPersistent) {
      e = dllm::launch_gemm_persistent(h->W, a.hidden, d, V, w.idx, w.ctr, h->cus, parts, st);
    } else {
      e = dllm::launch_gemm_large(h->W, a.hidden, d, V, w.idx, w.ctr, n_rt, plan.fixed_slices, parts, st);
    }
    if (h->log)
      fprintf(stderr, "[dllm] step B=%d rows<=%lld path=%s slices=%d cus=%d ext=%d score=%d threshold=%d\n",
              batched ? a.B : 0, (long long)rows_max,
              fused ? "small-find" : path == kSmall ? "small" : path == kPersistent ? "persistent" : "streaming",
              plan.fixed_slices, h->cus,
              (int)ext, pol.score, pol.use_threshold);
    if (e != hipSuccess) return hip_failed(h, "GEMM launch", e);
    if (h->ev_after) {
      const hipError_t er = hipEventRecord(h->ev_after, st);
      if (er != hipSuccess) return hip_failed(h, "hipEventRecord", er);
    }
    if (path == kSmall) {
      // merge (one workgroup per row), selection and commit of <= 32 rows
      const dllm::FewRowResults res = {w.row_tok, w.row_conf, w.row_lse, w.row_margin, w.row_entropy};
      const hipError_t ef = dllm::launch_finish_small(w.ctr, w.idx, req, a.B, a.L, k_stride, parts, pol, a.k, a.mask,
                                                      a.tokens, o, res, st);
      if (ef != hipSuccess) return hip_failed(h, "few-row finish launch", ef);
      return DLLM_OK;
    }
    // single sequence: the merge writes the row outputs; batched: it fills
    // the workspace rows and the selection copies each sequence's rows out
    dllm_step_out om = {};
    if (batched) {
      om.row_margin = w.row_margin;
      om.row_entropy = w.row_entropy;
    } else {
      om = o;
    }
    const hipError_t em = dllm::launch_merge(w.ctr, w.idx, parts, pol.score, (int)rows_max, w.row_tok, w.row_conf,
                                             w.row_lse, w.keys, om, st);
    if (em != hipSuccess) return hip_failed(h, "merge launch", em);
  }
  const hipError_t es = dllm::launch_topk_scatter(w.ctr, req, a.B, a.L, k_stride, a.k, pol, w, a.mask, a.tokens, o, st);
  if (es != hipSuccess) return hip_failed(h, "selection launch", es);
  return DLLM_OK;
}

}  // namespace

extern "C" {

const char* dllm_status_string(dllm_status s) {
  // A C caller may pass any int: read the argument's bits as an int rather
  // than as the C++ enum, whose valid range ends at the largest enumerator's
  // bit width (loading 99 as dllm_status is undefined behaviour).
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case DLLM_OK: return "ok";
    case DLLM_ERR_INVALID_ARG: return "invalid argument";
    case DLLM_ERR_UNSUPPORTED: return "unsupported argument (shape divisibility, pointer alignment or size limit)";
    case DLLM_ERR_WORKSPACE: return "workspace missing or too small";
    case DLLM_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t dllm_masked_readout_workspace_bytes(int64_t L_max, int64_t d, int64_t V, int32_t k_max) {
  if (!limits_ok(L_max, d, V, k_max)) return 0;
  return carve(L_max, V, nullptr, nullptr);
}

dllm_status dllm_masked_readout_create(dllm_readout** out, const uint16_t* W_lm, int64_t V, int64_t d,
                                       int64_t L_max, int32_t k_max, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (!out) return DLLM_ERR_INVALID_ARG;
  *out = nullptr;
  if (!W_lm) return DLLM_ERR_INVALID_ARG;
  if (k_max > DLLM_K_MAX_LIMIT) return DLLM_ERR_UNSUPPORTED;
  if (!limits_ok(L_max, d, V, k_max)) return DLLM_ERR_INVALID_ARG;
  if (d % 8 != 0 || !aligned16(W_lm)) return DLLM_ERR_UNSUPPORTED;
  const size_t need = carve(L_max, V, nullptr, nullptr);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign) != 0) return DLLM_ERR_WORKSPACE;

  dllm_readout* h = new (std::nothrow) dllm_readout;
  if (!h) return DLLM_ERR_HIP;
  h->W = W_lm;
  h->V = V;
  h->d = d;
  h->L_max = L_max;
  h->k_max = k_max;
  h->stream = reinterpret_cast<hipStream_t>(stream);
  h->cus = 0;  // queried at the first step
  h->slices_override = 0;
  h->ev_before = nullptr;
  h->ev_after = nullptr;
  const char* lg = getenv("DLLM_LOG");
  h->log = lg && lg[0] == '1';
  carve(L_max, V, reinterpret_cast<uint8_t*>(workspace), &h->ws);
  *out = h;
  return DLLM_OK;
}

dllm_status dllm_masked_readout_destroy(dllm_readout* h) {
  delete h;
  return DLLM_OK;
}

dllm_status dllm_masked_readout_set_slices(dllm_readout* h, int32_t slices) {
  if (!h || slices < 0 || slices > dllm::kMaxLargeSlices) return DLLM_ERR_INVALID_ARG;
  h->slices_override = slices;
  return DLLM_OK;
}

dllm_status dllm_masked_readout_set_gemm_events(dllm_readout* h, void* ev_before, void* ev_after) {
  if (!h || ((ev_before == nullptr) != (ev_after == nullptr))) return DLLM_ERR_INVALID_ARG;
  h->ev_before = reinterpret_cast<hipEvent_t>(ev_before);
  h->ev_after = reinterpret_cast<hipEvent_t>(ev_after);
  return DLLM_OK;
}

dllm_status dllm_masked_readout_step(dllm_readout* h, const uint16_t* hidden, int64_t L, uint8_t* mask,
                                     int32_t* tokens, int32_t k, int64_t win_lo, int64_t win_hi,
                                     int64_t block, const dllm_step_out* out) {
  return dllm_masked_readout_step_ex(h, hidden, L, mask, tokens, k, win_lo, win_hi, block, nullptr, out);
}

dllm_status dllm_masked_readout_step_ex(dllm_readout* h, const uint16_t* hidden, int64_t L, uint8_t* mask,
                                        int32_t* tokens, int32_t k, int64_t win_lo, int64_t win_hi,
                                        int64_t block, const dllm_policy* policy, const dllm_step_out* out) {
  if (!h || !hidden || !mask || !tokens) return DLLM_ERR_INVALID_ARG;
  dllm::Policy pol;
  const dllm_status ps = parse_policy(policy, &pol);
  if (ps != DLLM_OK) return ps;
  if (L <= 0 || L > h->L_max) return DLLM_ERR_INVALID_ARG;
  if (k < 0 || k > h->k_max) return DLLM_ERR_INVALID_ARG;
  if (win_lo < 0 || win_lo > win_hi || win_hi > L) return DLLM_ERR_INVALID_ARG;
  if (block < 0) return DLLM_ERR_INVALID_ARG;
  if (!aligned16(hidden)) return DLLM_ERR_UNSUPPORTED;
  dllm_step_out o = {};
  if (out) o = *out;
  const int64_t span = win_hi - win_lo;
  StepArgs a = {};
  a.hidden = hidden;
  a.L = L;
  a.mask = mask;
  a.tokens = tokens;
  a.block = block;
  a.k = k;
  a.win_lo = win_lo;
  a.win_hi = win_hi;
  a.seqs = nullptr;
  a.B = 1;
  a.rows_max = (block > 0 && block < span) ? block : span;
  a.hidden_rows = L;
  return run_step(h, a, pol, o);
}

dllm_status dllm_masked_readout_step_noalloc(const uint16_t* W_lm, int64_t V, int64_t d, const uint16_t* hidden,
                                             int64_t L, uint8_t* mask, int32_t* tokens, int32_t k, int64_t win_lo,
                                             int64_t win_hi, int64_t block, const dllm_policy* policy,
                                             const dllm_step_out* out, void* stream) {
  // the checks of create (limits L_max = L, k_max = k) ...
  if (!W_lm) return DLLM_ERR_INVALID_ARG;
  if (k > DLLM_K_MAX_LIMIT) return DLLM_ERR_UNSUPPORTED;
  if (!limits_ok(L, d, V, k)) return DLLM_ERR_INVALID_ARG;
  if (d % 8 != 0 || !aligned16(W_lm)) return DLLM_ERR_UNSUPPORTED;
  if (carve(L, V, nullptr, nullptr) > DLLM_NOALLOC_SCRATCH_BYTES) return DLLM_ERR_WORKSPACE;
  // ... and of the step, all before the first HIP call
  if (!hidden || !mask || !tokens) return DLLM_ERR_INVALID_ARG;
  dllm::Policy pol;
  const dllm_status ps = parse_policy(policy, &pol);
  if (ps != DLLM_OK) return ps;
  if (win_lo < 0 || win_lo > win_hi || win_hi > L) return DLLM_ERR_INVALID_ARG;
  if (block < 0) return DLLM_ERR_INVALID_ARG;
  if (!aligned16(hidden)) return DLLM_ERR_UNSUPPORTED;
  void* base = nullptr;
  const dllm_status ss = scratch_for_current_device(&base);
  if (ss != DLLM_OK) return ss;

  dllm_readout h;  // host object on the stack: nothing is allocated
  h.W = W_lm;
  h.V = V;
  h.d = d;
  h.L_max = L;
  h.k_max = k;
  h.stream = reinterpret_cast<hipStream_t>(stream);
  h.cus = 0;
  h.slices_override = 0;
  h.log = false;
  h.ev_before = nullptr;
  h.ev_after = nullptr;
  carve(L, V, reinterpret_cast<uint8_t*>(base), &h.ws);
  dllm_step_out o = {};
  if (out) o = *out;
  const int64_t span = win_hi - win_lo;
  StepArgs a = {};
  a.hidden = hidden;
  a.L = L;
  a.mask = mask;
  a.tokens = tokens;
  a.block = block;
  a.k = k;
  a.win_lo = win_lo;
  a.win_hi = win_hi;
  a.seqs = nullptr;
  a.B = 1;
  a.rows_max = (block > 0 && block < span) ? block : span;
  a.hidden_rows = L;
  return run_step(&h, a, pol, o);
}

dllm_status dllm_masked_readout_step_batch(dllm_readout* h, int32_t B, const uint16_t* hidden, int64_t L,
                                           uint8_t* mask, int32_t* tokens, const dllm_seq* seqs, int64_t block,
                                           const dllm_policy* policy, const dllm_step_out* out) {
  if (!h || !hidden || !mask || !tokens || !seqs) return DLLM_ERR_INVALID_ARG;
  dllm::Policy pol;
  const dllm_status ps = parse_policy(policy, &pol);
  if (ps != DLLM_OK) return ps;
  if (B < 1 || B > dllm::kBatchMax) return DLLM_ERR_INVALID_ARG;
  if (L <= 0 || L > h->L_max || (int64_t)B * L > h->L_max) return DLLM_ERR_INVALID_ARG;
  if (block < 0) return DLLM_ERR_INVALID_ARG;
  dllm::SeqTable tab;
  int64_t rows_max = 0;
  for (int b = 0; b < B; ++b) {
    const dllm_seq& q = seqs[b];
    if (q.k < 0 || q.k > h->k_max) return DLLM_ERR_INVALID_ARG;
    if (q.win_lo < 0 || q.win_lo > q.win_hi || (int64_t)q.win_hi > L) return DLLM_ERR_INVALID_ARG;
    const int64_t span = (int64_t)q.win_hi - q.win_lo;
    rows_max += (block > 0 && block < span) ? block : span;
    tab.lo[b] = q.win_lo;
    tab.hi[b] = q.win_hi;
    tab.k[b] = q.k;
  }
  for (int b = B; b < dllm::kBatchMax; ++b) tab.lo[b] = tab.hi[b] = tab.k[b] = 0;
  if (!aligned16(hidden)) return DLLM_ERR_UNSUPPORTED;
  dllm_step_out o = {};
  if (out) o = *out;
  StepArgs a = {};
  a.hidden = hidden;
  a.L = L;
  a.mask = mask;
  a.tokens = tokens;
  a.block = block;
  a.k = 0;
  a.seqs = &tab;
  a.B = B;
  a.rows_max = rows_max;
  a.hidden_rows = (int64_t)B * L;
  return run_step(h, a, pol, o);
}

}  // extern "C"
