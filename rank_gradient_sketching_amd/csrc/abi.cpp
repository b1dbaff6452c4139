// C ABI of the LoGRA hot path (declared in include/logra.h).
//
// Every entry point validates all of its arguments on the host before the
// first HIP call and returns a status code; nothing throws across the ABI.
#include "logra.h"

#include <math.h>
#include <stdio.h>

#include "internal.hpp"

namespace {

thread_local char g_hip_msg[256] = "";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return LOGRA_OK;
  snprintf(g_hip_msg, sizeof(g_hip_msg), "HIP error %d: %s", (int)e,
           hipGetErrorString(e));
  return LOGRA_EHIP;
}

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

static_assert(LOGRA_MAX_SHARED == logra::kMaxShared, "shared-output limit");
static_assert(LOGRA_MAX_GROUPS == logra::kMaxGroups, "input-group limit");
static_assert(LOGRA_MAX_LAYER_OUT == logra::kMaxOut, "outputs per call");
static_assert(LOGRA_MAX_MERGE == logra::kMaxMerge, "weights per merge call");
static_assert(LOGRA_NOALLOC_SCRATCH_BYTES == logra::kNoallocScratchBytes, "no-alloc scratch size");

constexpr int64_t kDimLimit = int64_t(1) << 31;
constexpr int64_t kDyStrideLimit = int64_t(1) << 26;

bool dim_ok(int64_t x) { return x >= 1 && x < kDimLimit; }
bool rank_ok(int32_t r) { return r >= 1 && r <= LOGRA_MAX_RANK; }
bool kind_ok(int kind) { return kind == LOGRA_RADEMACHER || kind == LOGRA_GAUSSIAN; }
// Row stride of a bf16 matrix: >= row length, multiple of 8 (16-byte rows).
bool ld_ok(int64_t ld, int64_t row) { return ld >= row && ld % 8 == 0 && ld < (int64_t(1) << 40); }

}  // namespace

extern "C" {

int logra_abi_version(void) { return LOGRA_ABI_VERSION; }

const char* logra_status_str(int status) {
  switch (status) {
    case LOGRA_OK:
      return "ok";
    case LOGRA_EINVAL:
      return "invalid argument";
    case LOGRA_EWORKSPACE:
      return "workspace (or the no-alloc scratch) missing or too small";
    case LOGRA_EHIP:
      return g_hip_msg[0] ? g_hip_msg : "HIP error";
    default:
      return "unknown status";
  }
}

int logra_regen_A(uint64_t seed, uint64_t stream, int kind, int32_t r,
                  int64_t k, float* A, hipStream_t s) {
  if (A == nullptr || !aligned(A, 4) || !rank_ok(r) || !dim_ok(k) || !kind_ok(kind))
    return LOGRA_EINVAL;
  return hip_status(logra::launch_regen(seed, stream, kind, r, k, A, s));
}

int logra_set_kernel_choice(int which, int mode) {
  return logra::set_kernel_choice(which, mode) ? LOGRA_OK : LOGRA_EINVAL;
}

size_t logra_sketch_ws_bytes(int64_t T, int64_t d, int64_t k, int32_t r) {
  logra::SketchPlan p{};
  if (!logra::make_sketch_plan(T, 1, &d, k, r, &p)) return 0;
  return p.total;
}

size_t logra_sketch_shared_ws_bytes(int64_t T, int64_t k, int32_t r, int32_t n_out,
                                    const int64_t* d) {
  if (d == nullptr || n_out < 1 || n_out > LOGRA_MAX_SHARED) return 0;
  logra::SketchPlan p{};
  if (!logra::make_sketch_plan(T, n_out, d, k, r, &p)) return 0;
  return p.total;
}

size_t logra_sketch_layer_ws_bytes(int64_t T, int32_t r, int32_t n_groups,
                                   const logra_sketch_group* groups) {
  if (groups == nullptr || n_groups < 1 || n_groups > LOGRA_MAX_GROUPS) return 0;
  int64_t k[LOGRA_MAX_GROUPS];
  int n_out[LOGRA_MAX_GROUPS];
  int64_t d[LOGRA_MAX_LAYER_OUT];
  int o = 0;
  for (int g = 0; g < n_groups; ++g) {
    k[g] = groups[g].k;
    n_out[g] = groups[g].n_out;
    if (n_out[g] < 1 || n_out[g] > LOGRA_MAX_SHARED || o + n_out[g] > LOGRA_MAX_LAYER_OUT)
      return 0;
    for (int i = 0; i < n_out[g]; ++i) d[o++] = groups[g].d[i];
  }
  logra::SketchPlan p{};
  if (!logra::make_sketch_plan_groups(T, n_groups, k, n_out, d, r, &p)) return 0;
  return p.total;
}

namespace {

// Checks shared by every sketch entry point; fills the plan.  T == 0 is
// reported as LOGRA_OK with *run = false.
constexpr int32_t kDeferFlags = LOGRA_SKETCH_DEFER | LOGRA_SKETCH_PENDING;

// The flags of a sketch call: OVERWRITE and the deferral flags; a deferred
// chain needs tokens in every call, and a deferring call writes no S, so it
// takes no overwrite flag.
int flags_check(int32_t flags, int64_t T, bool allow_defer) {
  if ((flags & ~(LOGRA_SKETCH_OVERWRITE | kDeferFlags)) != 0) return LOGRA_EINVAL;
  if ((flags & kDeferFlags) != 0) {
    if (!allow_defer || T < 1) return LOGRA_EINVAL;
    if ((flags & LOGRA_SKETCH_DEFER) && (flags & LOGRA_SKETCH_OVERWRITE)) return LOGRA_EINVAL;
  }
  return LOGRA_OK;
}

// S of every output: needed by the kernels, and by the zero fill at T == 0
// (a deferring call never touches S, but its S must still be a valid
// argument).  One accumulator per output: no two S ranges (d x r floats)
// overlap.
int outputs_s_check(const logra::SketchOut* outs, int n_out, int32_t r) {
  for (int o = 0; o < n_out; ++o) {
    if (outs[o].S == nullptr || !aligned(outs[o].S, 4)) return LOGRA_EINVAL;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(outs[o].S);
    const uintptr_t hi = lo + 4 * (uintptr_t)outs[o].d * (uintptr_t)r;
    for (int o2 = 0; o2 < o; ++o2) {
      const uintptr_t lo2 = reinterpret_cast<uintptr_t>(outs[o2].S);
      const uintptr_t hi2 = lo2 + 4 * (uintptr_t)outs[o2].d * (uintptr_t)r;
      if (lo < hi2 && lo2 < hi) return LOGRA_EINVAL;
    }
  }
  return LOGRA_OK;
}

// dY of every output (calls with tokens).
int outputs_dy_check(const logra::SketchOut* outs, int n_out) {
  for (int o = 0; o < n_out; ++o) {
    const logra::SketchOut& q = outs[o];
    if (q.dY == nullptr) return LOGRA_EINVAL;
    if (!aligned(q.dY, 16) || !ld_ok(q.ldd, q.d)) return LOGRA_EINVAL;
    // dY is read through 32-bit buffer offsets spanning 32 rows of 2 * ldd bytes
    if (q.ldd >= kDyStrideLimit) return LOGRA_EINVAL;
  }
  return LOGRA_OK;
}

int sketch_checks(const logra::SketchGroup* groups, int n_groups, int64_t T, int32_t r,
                  int kind, int32_t flags, const logra::SketchOut* outs, void* ws,
                  size_t ws_bytes, logra::SketchPlan* plan, bool* run,
                  bool allow_defer = true) {
  *run = false;
  if (n_groups < 1 || n_groups > LOGRA_MAX_GROUPS) return LOGRA_EINVAL;
  if (!rank_ok(r) || !kind_ok(kind)) return LOGRA_EINVAL;
  int st = flags_check(flags, T, allow_defer);
  if (st != LOGRA_OK) return st;
  int64_t k[LOGRA_MAX_GROUPS];
  int n_out_g[LOGRA_MAX_GROUPS];
  int64_t d[LOGRA_MAX_LAYER_OUT];
  int n_out = 0;
  for (int g = 0; g < n_groups; ++g) {
    if (!dim_ok(groups[g].k)) return LOGRA_EINVAL;
    if (groups[g].n_out < 1 || groups[g].n_out > LOGRA_MAX_SHARED) return LOGRA_EINVAL;
    if (n_out + groups[g].n_out > LOGRA_MAX_LAYER_OUT) return LOGRA_EINVAL;
    k[g] = groups[g].k;
    n_out_g[g] = groups[g].n_out;
    n_out += groups[g].n_out;
  }
  for (int o = 0; o < n_out; ++o) {
    if (!dim_ok(outs[o].d)) return LOGRA_EINVAL;
    d[o] = outs[o].d;
  }
  if (T < 0 || T >= kDimLimit) return LOGRA_EINVAL;
  if (T == 0 && (flags & LOGRA_SKETCH_OVERWRITE) == 0) return LOGRA_OK;
  st = outputs_s_check(outs, n_out, r);
  if (st != LOGRA_OK) return st;
  if (T == 0) {
    *run = true;
    return LOGRA_OK;
  }
  for (int g = 0; g < n_groups; ++g) {
    const logra::SketchGroup& q = groups[g];
    if (q.X == nullptr || !aligned(q.X, 16) || !ld_ok(q.ldx, q.k)) return LOGRA_EINVAL;
  }
  st = outputs_dy_check(outs, n_out);
  if (st != LOGRA_OK) return st;
  if (!logra::make_sketch_plan_groups(T, n_groups, k, n_out_g, d, r, plan)) return LOGRA_EINVAL;
  if (ws == nullptr || ws_bytes < plan->total || !aligned(ws, 256)) return LOGRA_EWORKSPACE;
  *run = true;
  return LOGRA_OK;
}

// After sketch_checks set *run: the zero fill of every output at T == 0 (the
// plan is not built then; n_out is the call's own output count), else the
// kernels.
int run_sketch(const logra::SketchPlan& p, const logra::SketchGroup* groups,
               const logra::SketchOut* outs, int n_out, int64_t T, int32_t r, int kind,
               int32_t flags, void* ws, hipStream_t s) {
  if (T == 0) return hip_status(logra::launch_zero_outputs(outs, n_out, r, s));
  return hip_status(logra::launch_sketch(p, groups, outs, (int)T, r, kind,
                                         (flags & LOGRA_SKETCH_OVERWRITE) != 0,
                                         (flags & LOGRA_SKETCH_DEFER) != 0,
                                         (flags & LOGRA_SKETCH_PENDING) != 0,
                                         static_cast<char*>(ws), s));
}

}  // namespace

int logra_sketch_accumulate(const uint16_t* X, int64_t ldx, const uint16_t* dY,
                            int64_t ldd, int64_t T, int64_t d, int64_t k,
                            int32_t r, uint64_t seed, uint64_t stream, int kind,
                            int32_t flags, float* S, void* ws, size_t ws_bytes,
                            hipStream_t s) {
  const logra::SketchGroup grp{X, ldx, k, seed, stream, 1};
  const logra::SketchOut out{dY, ldd, d, S};
  logra::SketchPlan p{};
  bool run = false;
  const int st = sketch_checks(&grp, 1, T, r, kind, flags, &out, ws, ws_bytes, &p, &run);
  if (st != LOGRA_OK || !run) return st;
  return run_sketch(p, &grp, &out, 1, T, r, kind, flags, ws, s);
}

int logra_sketch_accumulate_noalloc(const uint16_t* X, int64_t ldx, const uint16_t* dY,
                                    int64_t ldd, int64_t T, int64_t d, int64_t k, int32_t r,
                                    uint64_t seed, uint64_t stream, int kind, int32_t flags,
                                    float* S, hipStream_t s) {
  const logra::SketchGroup grp{X, ldx, k, seed, stream, 1};
  const logra::SketchOut out{dY, ldd, d, S};
  // every argument and the scratch size are checked before the first HIP call
  // (the scratch-address lookup); the checks see a stand-in workspace of the
  // full scratch size at a 256-byte-aligned address
  logra::SketchPlan p{};
  bool run = false;
  const int st = sketch_checks(&grp, 1, T, r, kind, flags, &out,
                               reinterpret_cast<void*>(uintptr_t(256)),
                               LOGRA_NOALLOC_SCRATCH_BYTES, &p, &run, /*allow_defer=*/false);
  if (st != LOGRA_OK || !run) return st;
  if (T == 0) return hip_status(logra::launch_zero_outputs(&out, 1, r, s));
  void* ws = nullptr;
  const int sh = hip_status(logra::noalloc_scratch(s, &ws));
  if (sh != LOGRA_OK) return sh;
  return run_sketch(p, &grp, &out, 1, T, r, kind, flags, ws, s);
}

int logra_sketch_accumulate_shared(const uint16_t* X, int64_t ldx, int64_t T, int64_t k,
                                   int32_t r, uint64_t seed, uint64_t stream, int kind,
                                   int32_t flags, int32_t n_out, const uint16_t* const* dY,
                                   const int64_t* ldd, const int64_t* d, float* const* S,
                                   void* ws, size_t ws_bytes, hipStream_t s) {
  if (n_out < 1 || n_out > LOGRA_MAX_SHARED) return LOGRA_EINVAL;
  if (dY == nullptr || ldd == nullptr || d == nullptr || S == nullptr) return LOGRA_EINVAL;
  const logra::SketchGroup grp{X, ldx, k, seed, stream, n_out};
  logra::SketchOut outs[LOGRA_MAX_SHARED];
  for (int o = 0; o < n_out; ++o) outs[o] = logra::SketchOut{dY[o], ldd[o], d[o], S[o]};
  logra::SketchPlan p{};
  bool run = false;
  const int st = sketch_checks(&grp, 1, T, r, kind, flags, outs, ws, ws_bytes, &p, &run);
  if (st != LOGRA_OK || !run) return st;
  return run_sketch(p, &grp, outs, n_out, T, r, kind, flags, ws, s);
}

int logra_sketch_accumulate_layer(int64_t T, int32_t r, int kind, int32_t flags,
                                  int32_t n_groups, const logra_sketch_group* groups, void* ws,
                                  size_t ws_bytes, hipStream_t s) {
  if (groups == nullptr || n_groups < 1 || n_groups > LOGRA_MAX_GROUPS) return LOGRA_EINVAL;
  logra::SketchGroup grp[LOGRA_MAX_GROUPS];
  logra::SketchOut outs[LOGRA_MAX_LAYER_OUT];
  int n_out = 0;
  for (int g = 0; g < n_groups; ++g) {
    const logra_sketch_group& q = groups[g];
    if (q.n_out < 1 || q.n_out > LOGRA_MAX_SHARED || n_out + q.n_out > LOGRA_MAX_LAYER_OUT)
      return LOGRA_EINVAL;
    grp[g] = logra::SketchGroup{q.X, q.ldx, q.k, q.seed, q.stream, q.n_out};
    for (int i = 0; i < q.n_out; ++i)
      outs[n_out++] = logra::SketchOut{q.dY[i], q.ldd[i], q.d[i], q.S[i]};
  }
  logra::SketchPlan p{};
  bool run = false;
  const int st = sketch_checks(grp, n_groups, T, r, kind, flags, outs, ws, ws_bytes, &p, &run);
  if (st != LOGRA_OK || !run) return st;
  return run_sketch(p, grp, outs, n_out, T, r, kind, flags, ws, s);
}

size_t logra_sketch_p_bytes(int64_t T, int32_t r) {
  const int64_t d = 1;
  logra::SketchPlan p{};
  if (!logra::make_sketch_plan(T, 1, &d, 1, r, &p)) return 0;
  return logra::plan_p_bytes(p);
}

size_t logra_sketch_project_ws_bytes(int64_t k, int32_t r) {
  const int64_t d = 1;
  logra::SketchPlan p{};
  if (!logra::make_sketch_plan(1, 1, &d, k, r, &p)) return 0;
  return logra::plan_gauss_bytes(p, 0);
}

int logra_sketch_project(const uint16_t* X, int64_t ldx, int64_t T, int64_t k, int32_t r,
                         uint64_t seed, uint64_t stream, int kind, uint16_t* P, size_t p_bytes,
                         void* ws, size_t ws_bytes, hipStream_t s) {
  if (!rank_ok(r) || !kind_ok(kind) || !dim_ok(k)) return LOGRA_EINVAL;
  if (T < 0 || T >= kDimLimit) return LOGRA_EINVAL;
  if (T == 0) return LOGRA_OK;
  if (X == nullptr || !aligned(X, 16) || !ld_ok(ldx, k)) return LOGRA_EINVAL;
  const int64_t d = 1;
  logra::SketchPlan p{};
  if (!logra::make_sketch_plan(T, 1, &d, k, r, &p)) return LOGRA_EINVAL;
  if (P == nullptr || !aligned(P, 16) || p_bytes < logra::plan_p_bytes(p)) return LOGRA_EINVAL;
  const bool gauss = kind == LOGRA_GAUSSIAN;
  if (gauss && (ws == nullptr || ws_bytes < logra::plan_gauss_bytes(p, 0) || !aligned(ws, 256)))
    return LOGRA_EWORKSPACE;
  const logra::SketchGroup g{X, ldx, k, seed, stream, 1};
  return hip_status(logra::launch_project_only(p, g, (int)T, r, kind, P,
                                               gauss ? static_cast<uint16_t*>(ws) : nullptr, s));
}

size_t logra_sketch_accumulate_p_ws_bytes(int64_t T, int32_t r, int32_t n_out, const int64_t* d) {
  if (d == nullptr || n_out < 1 || n_out > LOGRA_MAX_SHARED) return 0;
  logra::SketchPlan p{};
  if (!logra::make_sketch_plan(T, n_out, d, 1, r, &p)) return 0;
  return logra::plan_part_bytes(p);
}

int logra_sketch_accumulate_p(const uint16_t* P, size_t p_bytes, int64_t T, int32_t r,
                              int32_t flags, int32_t n_out, const uint16_t* const* dY,
                              const int64_t* ldd, const int64_t* d, float* const* S, void* ws,
                              size_t ws_bytes, hipStream_t s) {
  if (n_out < 1 || n_out > LOGRA_MAX_SHARED) return LOGRA_EINVAL;
  if (dY == nullptr || ldd == nullptr || d == nullptr || S == nullptr) return LOGRA_EINVAL;
  if (!rank_ok(r)) return LOGRA_EINVAL;
  int st = flags_check(flags, T, /*allow_defer=*/true);
  if (st != LOGRA_OK) return st;
  logra::SketchOut outs[LOGRA_MAX_SHARED];
  for (int o = 0; o < n_out; ++o) {
    if (!dim_ok(d[o])) return LOGRA_EINVAL;
    outs[o] = logra::SketchOut{dY[o], ldd[o], d[o], S[o]};
  }
  if (T < 0 || T >= kDimLimit) return LOGRA_EINVAL;
  if (T == 0 && (flags & LOGRA_SKETCH_OVERWRITE) == 0) return LOGRA_OK;
  st = outputs_s_check(outs, n_out, r);
  if (st != LOGRA_OK) return st;
  if (T == 0) return hip_status(logra::launch_zero_outputs(outs, n_out, r, s));
  st = outputs_dy_check(outs, n_out);
  if (st != LOGRA_OK) return st;
  logra::SketchPlan p{};
  if (!logra::make_sketch_plan(T, n_out, d, 1, r, &p)) return LOGRA_EINVAL;
  if (P == nullptr || !aligned(P, 16) || p_bytes < logra::plan_p_bytes(p)) return LOGRA_EINVAL;
  if (ws == nullptr || ws_bytes < logra::plan_part_bytes(p) || !aligned(ws, 256))
    return LOGRA_EWORKSPACE;
  return hip_status(logra::launch_accumulate_only(
      p, P, outs, (int)T, r, (flags & LOGRA_SKETCH_OVERWRITE) != 0,
      (flags & LOGRA_SKETCH_DEFER) != 0, (flags & LOGRA_SKETCH_PENDING) != 0,
      static_cast<float*>(ws), s));
}

namespace {

// Checks of one merge weight (shared by both merge entry points).
bool merge_item_ok(const logra::MergeItem& m, int32_t r) {
  if (m.W == nullptr || m.S == nullptr) return false;
  if (!dim_ok(m.d) || !dim_ok(m.k) || !rank_ok(r)) return false;
  if (!aligned(m.W, 16) || !aligned(m.S, 4) || !ld_ok(m.ldw, m.k)) return false;
  // one work-group per tile of at least 128 rows x 256 columns, flat grid
  return ((m.d + 127) / 128) * ((m.k + 255) / 256) < (int64_t(1) << 31);
}

}  // namespace

int logra_merge(uint16_t* W, int64_t ldw, const float* S, int64_t d, int64_t k,
                int32_t r, uint64_t seed, uint64_t stream, int kind, float alpha,
                float eta, hipStream_t s) {
  const logra::MergeItem m{W, ldw, S, d, k, seed, stream};
  if (!merge_item_ok(m, r) || !kind_ok(kind)) return LOGRA_EINVAL;
  if (!isfinite(alpha) || !isfinite(eta)) return LOGRA_EINVAL;
  return hip_status(logra::launch_merge(&m, 1, r, kind, alpha, eta, s));
}

int logra_merge_many(int32_t n, const logra_merge_item* items, int32_t r, int kind,
                     float alpha, float eta, hipStream_t s) {
  if (items == nullptr || n < 1 || n > LOGRA_MAX_MERGE) return LOGRA_EINVAL;
  if (!rank_ok(r) || !kind_ok(kind) || !isfinite(alpha) || !isfinite(eta)) return LOGRA_EINVAL;
  logra::MergeItem m[LOGRA_MAX_MERGE];
  int64_t tasks = 0;
  for (int i = 0; i < n; ++i) {
    const logra_merge_item& q = items[i];
    m[i] = logra::MergeItem{q.W, q.ldw, q.S, q.d, q.k, q.seed, q.stream};
    if (!merge_item_ok(m[i], r)) return LOGRA_EINVAL;
    tasks += ((q.d + 127) / 128) * ((q.k + 255) / 256);
  }
  if (tasks >= (int64_t(1) << 31)) return LOGRA_EINVAL;
  // W is written in place: no weight's rows may overlap another's, nor any S
  // (read while every W is written)
  for (int i = 0; i < n; ++i) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(m[i].W);
    const uintptr_t hi =
        lo + 2 * ((uintptr_t)(m[i].d - 1) * (uintptr_t)m[i].ldw + (uintptr_t)m[i].k);
    for (int j = 0; j < n; ++j) {
      const uintptr_t slo = reinterpret_cast<uintptr_t>(m[j].S);
      const uintptr_t shi = slo + 4 * (uintptr_t)m[j].d * (uintptr_t)r;
      if (slo < hi && lo < shi) return LOGRA_EINVAL;
      if (j < i) {
        const uintptr_t lo2 = reinterpret_cast<uintptr_t>(m[j].W);
        const uintptr_t hi2 =
            lo2 + 2 * ((uintptr_t)(m[j].d - 1) * (uintptr_t)m[j].ldw + (uintptr_t)m[j].k);
        if (lo < hi2 && lo2 < hi) return LOGRA_EINVAL;
      }
    }
  }
  return hip_status(logra::launch_merge(m, n, r, kind, alpha, eta, s));
}

int logra_sketch_update(int rule, const float* S, float* m, float* v, float* U,
                        int64_t d, int32_t r, float beta1, float beta2, float eps,
                        int64_t step, hipStream_t s) {
  if (rule != LOGRA_UPDATE_SGD && rule != LOGRA_UPDATE_MOMENTUM && rule != LOGRA_UPDATE_ADAM)
    return LOGRA_EINVAL;
  if (!dim_ok(d) || !rank_ok(r) || S == nullptr || U == nullptr) return LOGRA_EINVAL;
  const bool use_m = rule != LOGRA_UPDATE_SGD;
  const bool use_v = rule == LOGRA_UPDATE_ADAM;
  if ((use_m && m == nullptr) || (use_v && v == nullptr)) return LOGRA_EINVAL;
  const float* arr[4] = {S, use_m ? m : nullptr, use_v ? v : nullptr, U};
  for (const float* a : arr)
    if (a != nullptr && !aligned(a, 4)) return LOGRA_EINVAL;
  auto beta_ok = [](float b) { return isfinite(b) && b >= 0.0f && b < 1.0f; };
  if (use_m && !beta_ok(beta1)) return LOGRA_EINVAL;
  if (use_v && (!beta_ok(beta2) || !isfinite(eps) || eps < 0.0f || step < 1)) return LOGRA_EINVAL;
  // Overlaps: U may be S itself, and for momentum m itself; any other overlap
  // of the four d x r arrays (or a partial one) is rejected.
  const int64_t n = d * (int64_t)r;
  auto lo = [](const float* a) { return reinterpret_cast<uintptr_t>(a); };
  auto overlap = [&](const float* a, const float* b) {
    return a != nullptr && b != nullptr && lo(a) < lo(b) + 4 * (uintptr_t)n &&
           lo(b) < lo(a) + 4 * (uintptr_t)n;
  };
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j) {
      if (!overlap(arr[i], arr[j])) continue;
      const bool same = arr[i] == arr[j];
      const bool allowed =
          (j == 3 && i == 0) || (j == 3 && i == 1 && rule == LOGRA_UPDATE_MOMENTUM);
      if (!same || !allowed) return LOGRA_EINVAL;
    }
  double bc1 = 1.0, bc2 = 1.0;
  if (use_v) {
    bc1 = 1.0 - pow((double)beta1, (double)step);
    bc2 = 1.0 - pow((double)beta2, (double)step);
  }
  return hip_status(logra::launch_sketch_update(rule, S, m, v, U, n, beta1, beta2, eps,
                                                bc1, bc2, s));
}

size_t logra_kl_ws_bytes(int64_t n_tok, int64_t vocab) {
  if (!dim_ok(n_tok) || !dim_ok(vocab)) return 0;
  return (size_t)logra::round_up(n_tok * 4, 256);
}

int logra_predicted_kl(const uint16_t* z_cur, const uint16_t* z_prop,
                       int64_t n_tok, int64_t vocab, int64_t ld, float tau,
                       float kl_budget, float alpha_max, float* q_alpha_out,
                       float* kl_tok, void* ws, size_t ws_bytes, hipStream_t s) {
  if (z_cur == nullptr || z_prop == nullptr || q_alpha_out == nullptr) return LOGRA_EINVAL;
  if (!dim_ok(n_tok) || !dim_ok(vocab) || !ld_ok(ld, vocab)) return LOGRA_EINVAL;
  if (!aligned(z_cur, 16) || !aligned(z_prop, 16) || !aligned(q_alpha_out, 4))
    return LOGRA_EINVAL;
  if (kl_tok != nullptr && !aligned(kl_tok, 4)) return LOGRA_EINVAL;
  if (!isfinite(tau) || !(tau > 0.0f)) return LOGRA_EINVAL;
  if (!isfinite(kl_budget) || !(kl_budget > 0.0f)) return LOGRA_EINVAL;
  if (!isfinite(alpha_max) || !(alpha_max >= 0.0f)) return LOGRA_EINVAL;
  float* rows = kl_tok;
  if (rows == nullptr) {
    if (ws == nullptr || ws_bytes < logra_kl_ws_bytes(n_tok, vocab) || !aligned(ws, 256))
      return LOGRA_EWORKSPACE;
    rows = static_cast<float*>(ws);
  }
  return hip_status(logra::launch_kl(z_cur, z_prop, (int)n_tok, (int)vocab, ld, tau,
                                     kl_budget, alpha_max, q_alpha_out, rows, s));
}

size_t logra_kl_sweep_ws_bytes(int64_t n_tok, int32_t n_alpha) {
  if (!dim_ok(n_tok) || n_alpha < 1 || n_alpha > LOGRA_MAX_SWEEP) return 0;
  return (size_t)logra::round_up(n_tok * 4 * (int64_t)n_alpha, 256);
}

int logra_predicted_kl_sweep(const uint16_t* z, const uint16_t* delta, int64_t n_tok,
                             int64_t vocab, int64_t ld, const float* alphas,
                             int32_t n_alpha, float tau, const float* weight,
                             float* kl_mean, float* kl_tok, void* ws, size_t ws_bytes,
                             hipStream_t s) {
  if (z == nullptr || delta == nullptr || alphas == nullptr || kl_mean == nullptr)
    return LOGRA_EINVAL;
  if (!dim_ok(n_tok) || !dim_ok(vocab) || !ld_ok(ld, vocab)) return LOGRA_EINVAL;
  if (n_alpha < 1 || n_alpha > LOGRA_MAX_SWEEP) return LOGRA_EINVAL;
  // the multiplier-major per-row buffer is indexed with 32-bit row counts
  if ((int64_t)n_alpha * n_tok >= kDimLimit) return LOGRA_EINVAL;
  if (!aligned(z, 16) || !aligned(delta, 16) || !aligned(kl_mean, 4)) return LOGRA_EINVAL;
  if (weight != nullptr && !aligned(weight, 4)) return LOGRA_EINVAL;
  if (kl_tok != nullptr && !aligned(kl_tok, 4)) return LOGRA_EINVAL;
  if (!isfinite(tau) || !(tau > 0.0f)) return LOGRA_EINVAL;
  for (int i = 0; i < n_alpha; ++i)
    if (!isfinite(alphas[i])) return LOGRA_EINVAL;
  float* rows = kl_tok;
  if (rows == nullptr) {
    if (ws == nullptr || ws_bytes < logra_kl_sweep_ws_bytes(n_tok, n_alpha) || !aligned(ws, 256))
      return LOGRA_EWORKSPACE;
    rows = static_cast<float*>(ws);
  }
  return hip_status(logra::launch_kl_sweep(z, delta, (int)n_tok, (int)vocab, ld, alphas,
                                           n_alpha, tau, weight, kl_mean, rows, s));
}

}  // extern "C"
