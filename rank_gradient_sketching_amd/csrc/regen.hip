// logra_regen_A kernels: write the projection A (r x k fp32) exactly as the
// sketch and merge kernels regenerate it on the fly.
//
// [LoGRA] (wispaper.ai summary of "LoGRA: Scaling LLM Reinforcement Learning
// with Low-Rank Gradient Sketches"), section Sketch: A is r x k, fixed while S
// accumulates, entries random signs scaled by 1/sqrt(r) by default; section
// Sync: the rollout side rebuilds A from the seed; section Rank: refreshed
// and Gaussian bases.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace logra {

// One wave per (row i, 256-column sign block); lane l writes columns
// 256 g + 4 l .. +3, whose signs are bits 4 l .. 4 l + 3 of the block.
__global__ __launch_bounds__(256) void regen_sign_kernel(uint64_t seed,
                                                         uint64_t stream, int r,
                                                         int64_t k, float c,
                                                         float* __restrict__ A) {
  const int64_t n_groups = (k + 255) >> 8;
  const int64_t wave_id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave_id >= (int64_t)r * n_groups) return;
  const int64_t row = wave_id / n_groups;
  const int64_t g = wave_id % n_groups;
  const int lane = threadIdx.x & 63;
  const Words4 b = sign_block(seed, stream, (uint64_t)g, (uint64_t)row);
  const uint64_t w = b.w[lane >> 4];
  const int64_t j0 = g * 256 + 4 * lane;
  float* out = A + row * k;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int bit = (int)((w >> ((4 * lane + e) & 63)) & 1u);
    if (j0 + e < k) out[j0 + e] = bit ? -c : c;
  }
}

// One thread per (row i, 4-column Gaussian group q).
__global__ __launch_bounds__(256) void regen_gauss_kernel(uint64_t seed,
                                                          uint64_t stream, int r,
                                                          int64_t k, float cr,
                                                          float* __restrict__ A) {
  const int64_t n_groups = (k + 3) >> 2;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)r * n_groups) return;
  const int64_t row = id / n_groups;
  const int64_t q = id % n_groups;
  uint16_t v[4];
  gaussian_entries_bf16(seed, stream, (uint64_t)q, (uint64_t)row, cr, v);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    if (4 * q + a < k) A[row * k + 4 * q + a] = bf16_to_f32(v[a]);
  }
}

float sign_scale(int r) { return (float)(1.0 / sqrt((double)r)); }

hipError_t launch_regen(uint64_t seed, uint64_t stream, int kind, int r,
                        int64_t k, float* A, hipStream_t s) {
  const float c = sign_scale(r);
  if (kind == 0) {
    const int64_t waves = (int64_t)r * ((k + 255) >> 8);
    const int64_t blocks = (waves + 3) / 4;
    hipLaunchKernelGGL(regen_sign_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       s, seed, stream, r, k, c, A);
  } else {
    const int64_t threads = (int64_t)r * ((k + 3) >> 2);
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(regen_gauss_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       s, seed, stream, r, k, c, A);
  }
  return hipGetLastError();
}

}  // namespace logra
