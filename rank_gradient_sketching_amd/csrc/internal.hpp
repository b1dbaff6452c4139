// Host-side plans and kernel launchers of the LoGRA hot path (internal; the
// public boundary is include/logra.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace logra {

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Projections that share the layer input X (and so, with the same seed, the
// same A) can be sketched together: one projection pass, one accumulate
// launch over all of their d groups.  A call takes up to kMaxGroups such input
// groups (a decoder layer's q/k/v, o, gate/up and down) with up to kMaxOut
// outputs in all: one projection launch over every group's token blocks, one
// accumulate launch over every output's d groups.
constexpr int kMaxShared = 4;
constexpr int kMaxGroups = 4;
constexpr int kMaxOut = 8;

// One output of a sketch call: S (d x r, fp32) += dY^T P.
struct SketchOut {
  const uint16_t* dY;
  int64_t ldd;
  int64_t d;
  float* S;
};

// One input group of a sketch call: P = X A^T with A from (seed, stream),
// feeding the group's n_out outputs (consecutive in the call's output list).
struct SketchGroup {
  const uint16_t* X;
  int64_t ldx;
  int64_t k;
  uint64_t seed;
  uint64_t stream;
  int n_out;
};

// Tiling of one sketch call (one or several outputs sharing X).  Both the
// workspace-size query and the launcher derive everything from this one
// function, so they agree.
struct SketchPlan {
  int rp;           // r padded to the accumulate kernel's N tiling (16..256)
  int p_rows;       // rows of the projected-input buffers (>= 32, >= rp)
  int nb32;         // 32-row blocks of A handled by the projection kernel
  int q_cols;       // d columns per lane in the accumulate kernel
  int64_t t_pad;    // T rounded up to 32 (one MFMA K step of tokens)
  int steps;        // t_pad / 32
  int n_groups;     // input groups
  int64_t k_pad[kMaxGroups];   // each group's k rounded up to 256 (one sign block)
  int out_off[kMaxGroups + 1]; // first output of each group
  int n_out;        // outputs, all groups together
  int dg_off[kMaxOut + 1];     // first d group of each output (prefix sums)
  int n_dgroups;    // 128-column d groups, all outputs together
  bool acc_wide;    // accumulate_wide_kernel (r >= 128) instead of accumulate_kernel
  int wg_groups;    // d groups per accumulate work-group (1, or 8 / (rp / 64) when wide)
  int wg_off[kMaxOut + 1];     // first accumulate work-group along d of each output
  int n_wg;         // accumulate work-groups along d, all outputs together
  int n_split;      // accumulate work-groups along T
  int steps_per_split;
  int64_t d_pad;    // n_dgroups * 16 * q_cols
  // workspace: each group's P (and Gaussian basis), the partial tiles
  size_t off_pt[kMaxGroups], off_gauss[kMaxGroups], off_part, total;
};

// n_groups input groups with k[g] columns and n_out[g] outputs each; d lists
// the outputs' row counts, group by group.
bool make_sketch_plan_groups(int64_t T, int n_groups, const int64_t* k, const int* n_out,
                             const int64_t* d, int r, SketchPlan* p);

// One input group with n_out outputs.
inline bool make_sketch_plan(int64_t T, int n_out, const int64_t* d, int64_t k, int r,
                             SketchPlan* p) {
  return make_sketch_plan_groups(T, 1, &k, &n_out, d, r, p);
}

// Process-wide kernel-choice override (which: 0 projection tile, 1 wide
// accumulate; mode: -1 automatic, 0 never, 1 always).  False on bad input.
bool set_kernel_choice(int which, int mode);

// Size of the library-owned scratch of logra_sketch_accumulate_noalloc.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;

// Device address of that scratch on the device of stream s (the current
// device for the null stream); looked up once per device, then cached.
hipError_t noalloc_scratch(hipStream_t s, void** ptr);

// c = 1/sqrt(r) computed in double and rounded once to float.
float sign_scale(int r);

hipError_t launch_regen(uint64_t seed, uint64_t stream, int kind, int r,
                        int64_t k, float* A, hipStream_t s);

// overwrite: S = dY^T (X A^T) instead of S += (S is not read).  defer: the
// result stays in the workspace's partial tiles and S is left alone;
// pending: the partial tiles hold earlier deferred results (same plan), which
// are added.  groups: p.n_groups entries; outs: p.n_out entries, group by
// group.
hipError_t launch_sketch(const SketchPlan& p, const SketchGroup* groups, const SketchOut* outs,
                         int T, int r, int kind, bool overwrite, bool defer, bool pending,
                         char* ws, hipStream_t s);

// Bytes of one input group's projected input P (bf16 hi and lo parts of
// t_pad x rp values), of its Gaussian basis (bf16, p_rows x k_pad) and of the
// partial tiles, as laid out in a call's workspace.
inline size_t plan_p_bytes(const SketchPlan& p) { return (size_t)2 * p.rp * (size_t)p.t_pad * 2; }
inline size_t plan_gauss_bytes(const SketchPlan& p, int g) {
  return (size_t)p.p_rows * (size_t)p.k_pad[g] * 2;
}
inline size_t plan_part_bytes(const SketchPlan& p) {
  return (size_t)p.n_split * p.d_pad * p.rp * 4;
}

// The two halves of launch_sketch for one input group, with P in a buffer of
// the caller's: the projection P = X A^T (gauss_ws: plan_gauss_bytes(p, 0)
// bytes for the Gaussian basis, unused for signs), and the accumulation of
// p.n_out outputs from such a P (part: plan_part_bytes(p) bytes).  Together
// they run the kernels of launch_sketch on the same plan, so the results are
// the same bits.
hipError_t launch_project_only(const SketchPlan& p, const SketchGroup& g, int T, int r, int kind,
                               uint16_t* P, uint16_t* gauss_ws, hipStream_t s);
hipError_t launch_accumulate_only(const SketchPlan& p, const uint16_t* P, const SketchOut* outs,
                                  int T, int r, bool overwrite, bool defer, bool pending,
                                  float* part, hipStream_t s);

// S = 0 for n_out outputs of d x r floats (a fill kernel, no memset node).
hipError_t launch_zero_outputs(const SketchOut* outs, int n_out, int r, hipStream_t s);

// One weight of a merge call: W (d x k bf16, row stride ldw) -= alpha eta S A
// with A from (seed, stream).
struct MergeItem {
  uint16_t* W;
  int64_t ldw;
  const float* S;
  int64_t d;
  int64_t k;
  uint64_t seed;
  uint64_t stream;
};
constexpr int kMaxMerge = 8;

// n items (1..kMaxMerge) with one rank and basis kind, in one launch.
hipError_t launch_merge(const MergeItem* items, int n, int r, int kind, float alpha,
                        float eta, hipStream_t s);

hipError_t launch_kl(const uint16_t* zc, const uint16_t* zp, int n_tok,
                     int vocab, int64_t ld, float tau, float kl_budget,
                     float alpha_max, float* q_alpha, float* kl_tok,
                     hipStream_t s);

// alphas: host array of n_alpha (1..LOGRA_MAX_SWEEP) multipliers; kl_tok:
// device float[n_alpha x n_tok] (written), kl_mean: device float[n_alpha].
hipError_t launch_kl_sweep(const uint16_t* z, const uint16_t* dz, int n_tok, int vocab,
                           int64_t ld, const float* alphas, int n_alpha, float tau,
                           const float* weight, float* kl_mean, float* kl_tok,
                           hipStream_t s);

// Sketch-space update rules (U from S and the optimizer state).
constexpr int kUpdateSgd = 0;
constexpr int kUpdateMomentum = 1;
constexpr int kUpdateAdam = 2;

// n = d r entries; bc1, bc2 = 1 - beta^t (Adam only).
hipError_t launch_sketch_update(int rule, const float* S, float* m, float* v, float* U,
                                int64_t n, float beta1, float beta2, float eps,
                                double bc1, double bc2, hipStream_t s);

}  // namespace logra
