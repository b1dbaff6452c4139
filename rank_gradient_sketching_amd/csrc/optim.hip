// logra_sketch_update kernel: the update factor U of W <- W - alpha eta U A
// from the sketch S and the state of a sketch-space optimizer.
//
// [LoGRA] (wispaper.ai summary of "LoGRA: Scaling LLM Reinforcement Learning
// with Low-Rank Gradient Sketches"), section Sketch: U equals S in the basic
// SGD variant; stateful sketch optimizers keep state of their own, which the
// pages do not define.  The stateful rules here are the textbook ones applied
// entrywise to the d x r sketch: heavy-ball momentum, and Adam (Kingma & Ba,
// ICLR 2015, Algorithm 1).
//
// One pass over d x r fp32 arrays (HBM-bound, a few MiB per layer): each
// thread reads S (and m, v), writes the state back and writes U, four
// entries at a time when every array is 16-byte aligned and d r % 4 == 0.
#include "common.hpp"
#include "internal.hpp"

namespace logra {

namespace {

struct UpdateArgs {
  const float* S;
  float* m;
  float* v;
  float* U;
  int64_t n;
  float b1, b2, eps;
  float bc1, bc2;   // 1 - b1^t, 1 - b2^t (Adam bias corrections)
};

template <int RULE>
__device__ __forceinline__ float update_one(float s, float* m, float* v, const UpdateArgs& a) {
  if constexpr (RULE == kUpdateMomentum) {
    const float mn = a.b1 * *m + s;
    *m = mn;
    return mn;
  } else if constexpr (RULE == kUpdateAdam) {
    const float mn = a.b1 * *m + (1.0f - a.b1) * s;
    const float vn = a.b2 * *v + (1.0f - a.b2) * (s * s);
    *m = mn;
    *v = vn;
    return (mn / a.bc1) / (sqrtf(vn / a.bc2) + a.eps);
  } else {
    return s;
  }
}

template <int RULE, bool VEC>
__global__ __launch_bounds__(256) void sketch_update_kernel(UpdateArgs a) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  if constexpr (VEC) {
    const int64_t n4 = a.n >> 2;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n4; q += stride) {
      const f32x4 s = reinterpret_cast<const f32x4*>(a.S)[q];
      f32x4 m = {0.f, 0.f, 0.f, 0.f}, v = {0.f, 0.f, 0.f, 0.f}, u;
      if (RULE != kUpdateSgd) m = reinterpret_cast<const f32x4*>(a.m)[q];
      if (RULE == kUpdateAdam) v = reinterpret_cast<const f32x4*>(a.v)[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float me = m[e], ve = v[e];
        u[e] = update_one<RULE>(s[e], &me, &ve, a);
        m[e] = me;
        v[e] = ve;
      }
      if (RULE != kUpdateSgd) reinterpret_cast<f32x4*>(a.m)[q] = m;
      if (RULE == kUpdateAdam) reinterpret_cast<f32x4*>(a.v)[q] = v;
      reinterpret_cast<f32x4*>(a.U)[q] = u;
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < a.n; i += stride) {
      float me = RULE != kUpdateSgd ? a.m[i] : 0.f;
      float ve = RULE == kUpdateAdam ? a.v[i] : 0.f;
      const float u = update_one<RULE>(a.S[i], &me, &ve, a);
      if (RULE != kUpdateSgd) a.m[i] = me;
      if (RULE == kUpdateAdam) a.v[i] = ve;
      a.U[i] = u;
    }
  }
}

template <int RULE>
void launch_rule(const UpdateArgs& a, bool vec, hipStream_t s) {
  const int64_t items = vec ? a.n >> 2 : a.n;
  int64_t blocks = (items + 255) / 256;
  if (blocks > 2048) blocks = 2048;   // grid-stride beyond eight work-groups per CU
  if (vec)
    hipLaunchKernelGGL((sketch_update_kernel<RULE, true>), dim3((unsigned)blocks), dim3(256), 0, s,
                       a);
  else
    hipLaunchKernelGGL((sketch_update_kernel<RULE, false>), dim3((unsigned)blocks), dim3(256), 0,
                       s, a);
}

}  // namespace

hipError_t launch_sketch_update(int rule, const float* S, float* m, float* v, float* U,
                                int64_t n, float beta1, float beta2, float eps,
                                double bc1, double bc2, hipStream_t s) {
  if (rule == kUpdateSgd && U == S) return hipSuccess;   // U = S in place: nothing to do
  UpdateArgs a{S, m, v, U, n, beta1, beta2, eps, (float)bc1, (float)bc2};
  auto al16 = [](const void* p) {
    return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0;
  };
  const bool vec = (n % 4) == 0 && al16(S) && al16(m) && al16(v) && al16(U);
  switch (rule) {
    case kUpdateSgd: launch_rule<kUpdateSgd>(a, vec, s); break;
    case kUpdateMomentum: launch_rule<kUpdateMomentum>(a, vec, s); break;
    default: launch_rule<kUpdateAdam>(a, vec, s); break;
  }
  return hipGetLastError();
}

}  // namespace logra
