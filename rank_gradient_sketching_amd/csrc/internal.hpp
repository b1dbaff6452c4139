// Host-side plans and kernel launchers of the LoGRA hot path (internal; the
// public boundary is include/logra.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace logra {

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Tiling of one logra_sketch_accumulate call.  Both the workspace-size query
// and the launcher derive everything from this one function, so they agree.
struct SketchPlan {
  int rp;           // r padded to the accumulate kernel's N tiling (16..256)
  int p_rows;       // rows of the projected-input buffers (>= 32, >= rp)
  int nb32;         // 32-row blocks of A handled by the projection kernel
  int q_cols;       // d columns per lane in the accumulate kernel
  int64_t t_pad;    // T rounded up to 32 (one MFMA K step of tokens)
  int64_t k_pad;    // k rounded up to 256 (one sign block)
  int steps;        // t_pad / 32
  int n_dgroups;    // accumulate work-groups along d
  int n_split;      // accumulate work-groups along T
  int steps_per_split;
  int64_t d_pad;    // n_dgroups * 16 * q_cols
  size_t off_pt, off_part, off_gauss, total;
};

bool make_sketch_plan(int64_t T, int64_t d, int64_t k, int r, SketchPlan* p);

// c = 1/sqrt(r) computed in double and rounded once to float.
float sign_scale(int r);

hipError_t launch_regen(uint64_t seed, uint64_t stream, int kind, int r,
                        int64_t k, float* A, hipStream_t s);

hipError_t launch_sketch(const SketchPlan& p, const uint16_t* X, int64_t ldx,
                         const uint16_t* dY, int64_t ldd, int T, int d, int k,
                         int r, uint64_t seed, uint64_t stream, int kind,
                         float* S, char* ws, hipStream_t s);

hipError_t launch_merge(uint16_t* W, int64_t ldw, const float* S, int d, int k,
                        int r, uint64_t seed, uint64_t stream, int kind,
                        float alpha, float eta, hipStream_t s);

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

}  // namespace logra
