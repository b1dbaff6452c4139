// logra_predicted_kl: q(D) = mean_t KL(softmax(z_cur[t]/tau) || softmax(z_prop[t]/tau))
// and the controller's alpha = min(alpha_max, sqrt(delta / q)), on gfx950.
//
// [LoGRA] (wispaper.ai summary of "LoGRA: Scaling LLM Reinforcement Learning
// with Low-Rank Gradient Sketches"), section PKL: before applying an update
// the method compares, on a small sample of responses and at one common
// temperature, the current vocabulary distribution with the one after the
// proposed update; the mean predicted KL scales as alpha^2 q(D) and the
// controller sets alpha = min(alpha_max, sqrt(delta / q(D))).
//
// One pass over both logit rows, no second read.  With a = z/tau,
// d = (z' - z - c)/tau and p = softmax(a):
//   KL = log E_p[e^d] - E_p[d] = E_p[g] + (log1p(x) - x),
//   g(d) = e^d - 1 - d >= 0,   x = E_p[e^d - 1] = E_p[d] + E_p[g].
// Each thread keeps (m, s, u1, u3) = (running max of a in log2 units,
// sum w, sum w d, sum w g) with w = 2^(a log2e - m); g comes from its Taylor
// polynomial for |d| <= 1/2 (no cancellation) and from exp otherwise.  The
// states merge by rescaling to the larger max (DPP/shuffle inside a wave,
// LDS across waves).  Per-row KL goes to kl_tok (or the workspace); a second
// one-work-group kernel averages the rows in a fixed order in fp64 and
// applies the controller.
// c is a per-row reference, the mean of z' - z over the row's first
// min(V, 64) elements (each wave forms the same value by a butterfly sum).
// The KL does not change when a constant is added to every z' - z of a row,
// so c changes nothing in exact arithmetic; it keeps a common offset of the
// proposed logits (a shift of the whole row, e.g. a bias-like update) out of
// g, whose fp32 sums would otherwise carry e^c - 1 - c and cancel against
// log1p(x) - x (an offset of -3 had cost ~40 % of a row's KL).
// Masked tokens: a logit of -inf is a token of probability zero.  Such a
// token of the current row adds nothing to the KL, and one with a finite
// current logit but a -inf proposed logit (p > 0, p' = 0) makes the row's
// KL +inf.  The first pass over a row does not look for them (z' - z is NaN
// or infinite there and leaves some sum of the state non-finite); a row
// whose merged state is not finite is read a second time in masked mode,
// which leaves the tokens with p = 0 out of the expectations (their
// proposed mass, when p' > 0, still enters the proposal's normaliser), notes
// those with p > 0 and p' = 0, and takes the row reference from the tokens
// where neither logit is -inf.  Rows of finite logits pay one check; NaN and
// +inf logits still give NaN.
// The reference itself is checked the same way: a row whose KL came out as
// a small difference of large terms (the first 64 tokens missed an offset
// the rest of the row carries) is read again about the p-weighted mean of
// z' - z, which its state already holds (see amplified).
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace logra {

namespace {

constexpr int kKlThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct KlState {
  float m, s, u1, u3;
};

__device__ __forceinline__ KlState kl_merge(KlState a, KlState b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return a;
  const float fa = a.m == -INFINITY ? 0.0f : exp2f(a.m - M);
  const float fb = b.m == -INFINITY ? 0.0f : exp2f(b.m - M);
  KlState o;
  o.m = M;
  o.s = a.s * fa + b.s * fb;
  o.u1 = a.u1 * fa + b.u1 * fb;
  o.u3 = a.u3 * fa + b.u3 * fb;
  return o;
}

// e^d - 1 - d.  For |d| <= 1/2 the Taylor series d^2 (1/2 + d/6 + d^2/24 +
// d^3/120 + d^4/720 + d^5/5040) has relative truncation error below 4e-6.
__device__ __forceinline__ float excess_exp(float d) {
  float p = 1.0f / 5040.0f;
  p = fmaf(p, d, 1.0f / 720.0f);
  p = fmaf(p, d, 1.0f / 120.0f);
  p = fmaf(p, d, 1.0f / 24.0f);
  p = fmaf(p, d, 1.0f / 6.0f);
  p = fmaf(p, d, 0.5f);
  float g = d * d * p;
  if (__builtin_expect(fabsf(d) > 0.5f, 0)) g = expf(d) - 1.0f - d;
  return g;
}

// Adds n (<= 8) elements to the state; z and zq are bf16 pairs, dref the
// row's reference difference.  MASK (the second pass): `hit` notes a token
// with p > 0 and p' = 0; a token with p = 0 adds nothing to s, u1 or the
// excess, but when p' > 0 it still belongs to the proposal's normaliser:
// with R = sum over such tokens of e^((z' - c)/tau) / sum_p>0 e^(z/tau),
// KL = log(E_p[e^d] + R) - E_p[d], so R joins u3 (as 2^(b - m) with
// b = (z' - c) log2e / tau, which also joins the running max).  The
// `b_of` lambda below forms b.
template <bool MASK>
__device__ __forceinline__ void kl_group(KlState& st, bool& hit, const float* z,
                                         const float* zq, int n, float l2t,
                                         float inv_tau, float dref) {
  float a2[8], dd[8];
  float cmax = -INFINITY;
  // b: the scaled proposed logit of a token with p = 0 and p' > 0 (-inf
  // otherwise); formed again where it is added, rather than held in eight
  // more registers
  auto b_of = [&](int e) {
    return e < n && z[e] == -INFINITY && zq[e] != -INFINITY ? (zq[e] - dref) * l2t : -INFINITY;
  };
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a2[e] = e < n ? z[e] * l2t : -INFINITY;
    if constexpr (MASK) {
      const bool pz = z[e] == -INFINITY, pq = zq[e] == -INFINITY;
      if (e < n && pq && !pz) hit = true;
      dd[e] = e < n && !pz && !pq ? ((zq[e] - z[e]) - dref) * inv_tau : 0.0f;
      cmax = fmaxf(cmax, b_of(e));
    } else {
      dd[e] = e < n ? ((zq[e] - z[e]) - dref) * inv_tau : 0.0f;
    }
    cmax = fmaxf(cmax, a2[e]);
  }
  if (cmax > st.m) {
    const float f = st.m == -INFINITY ? 0.0f : exp2f(st.m - cmax);
    st.s *= f;
    st.u1 *= f;
    st.u3 *= f;
    st.m = cmax;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // (a masked token, p = 0, is skipped outright: while a thread has seen
    // nothing else its running max is -inf, and 2^(-inf - -inf) is NaN)
    if (e < n && (!MASK || a2[e] != -INFINITY)) {
      const float w = exp2_normal(a2[e] - st.m);
      st.s += w;
      st.u1 = fmaf(w, dd[e], st.u1);
      st.u3 = fmaf(w, excess_exp(dd[e]), st.u3);
    }
    if constexpr (MASK) {
      const float b = b_of(e);
      if (b != -INFINITY) st.u3 += exp2_normal(b - st.m);
    }
  }
}

// Mean of zq - z over the first min(V, 64) elements of a row: lane l takes
// element l, then a butterfly sum.  Every lane (and every wave of the row)
// ends with the same bits: each level adds the same two partial sums, and
// fp32 addition is commutative.  MASK: over the tokens among them where
// neither logit is -inf (0 when there is none).
template <bool MASK>
__device__ __forceinline__ float row_reference(const uint16_t* a, const uint16_t* b, int V) {
  const int lane = threadIdx.x & 63;
  const int nref = V < 64 ? V : 64;
  if constexpr (MASK) {
    const float za = lane < nref ? bf16_to_f32(a[lane]) : 0.0f;
    const float zb = lane < nref ? bf16_to_f32(b[lane]) : 0.0f;
    const bool ok = lane < nref && za != -INFINITY && zb != -INFINITY;
    float x = ok ? zb - za : 0.0f;
    float cnt = ok ? 1.0f : 0.0f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      x += __shfl_xor(x, off);
      cnt += __shfl_xor(cnt, off);
    }
    return cnt > 0.0f ? x / cnt : 0.0f;
  } else {
    float x = lane < nref ? bf16_to_f32(b[lane]) - bf16_to_f32(a[lane]) : 0.0f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x / (float)nref;
  }
}

__device__ __forceinline__ bool state_finite(const KlState& t) {
  return isfinite(t.s) && isfinite(t.u1) && isfinite(t.u3);
}

// One pass over a row with reference difference dref: this thread's
// elements, then the wave's butterfly (every lane ends with the wave's state).
template <bool MASK>
__device__ __forceinline__ KlState kl_row_pass(const uint16_t* a, const uint16_t* b, int V,
                                               float l2t, float inv_tau, float dref, bool& hit) {
  KlState st{-INFINITY, 0.0f, 0.0f, 0.0f};
  // logits are read once: non-temporal loads (5 % faster over 65536 x 152064)
  const int nfull = V >> 3;
  for (int c = threadIdx.x; c < nfull; c += kKlThreads) {
    const u32x4 va = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a + 8 * c));
    const u32x4 vb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b + 8 * c));
    float z[8], zq[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      z[2 * p] = bf16_lo(va[p]);
      z[2 * p + 1] = bf16_hi(va[p]);
      zq[2 * p] = bf16_lo(vb[p]);
      zq[2 * p + 1] = bf16_hi(vb[p]);
    }
    kl_group<MASK>(st, hit, z, zq, 8, l2t, inv_tau, dref);
  }
  const int tail = V - 8 * nfull;
  if (tail > 0 && (int)threadIdx.x == nfull % kKlThreads) {
    float z[8], zq[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      z[e] = e < tail ? bf16_to_f32(a[8 * nfull + e]) : 0.0f;
      zq[e] = e < tail ? bf16_to_f32(b[8 * nfull + e]) : 0.0f;
    }
    kl_group<MASK>(st, hit, z, zq, tail, l2t, inv_tau, dref);
  }
  // wave reduction (fixed butterfly)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    KlState o;
    o.m = __shfl_xor(st.m, off);
    o.s = __shfl_xor(st.s, off);
    o.u1 = __shfl_xor(st.u1, off);
    o.u3 = __shfl_xor(st.u3, off);
    st = kl_merge(st, o);
  }
  return st;
}

// A row is read once more, re-centred, when its KL came out as a small
// difference of large terms.  With the reference c near the p-weighted mean
// of z' - z, E_p[g] is about the KL (both ~ Var_p(d) / 2 on small steps); an
// offset of the proposal that the row's first 64 tokens do not share leaves
// E_p[d] far from 0, E_p[g] ~ E_p[d^2] / 2 = (Var_p(d) + E_p[d]^2) / 2, and
// the fp32 sums' rounding enlarged by E_p[g] / KL.  The pass is repeated
// when that ratio exceeds 8, the KL estimated from the same state in fp32
// (rough exactly when the ratio is large, which is all the test needs).  The
// state already holds the fix: E_p[d] = u1 / s, so the next pass takes
// c + tau u1 / s.
__device__ __forceinline__ bool amplified(const KlState& t) {
  const float e1 = t.u1 / t.s, g = t.u3 / t.s;
  const float x = e1 + g;
  return g > 8.0f * (g + (log1pf(x) - x));
}

// The four wave states merged in order; every thread that calls this gets
// the same bits, so choices made on the result are work-group uniform.
__device__ __forceinline__ KlState merged_state(const KlState* wst) {
  KlState t = wst[0];
#pragma unroll
  for (int w = 1; w < kKlThreads / 64; ++w) t = kl_merge(t, wst[w]);
  return t;
}

// (eight work-groups per CU, i.e. eight waves per SIMD: the one-pass loop
// needs ~50 VGPRs, and the second pass, which would take ~70, spills a few
// registers instead; measured ~3 % faster than seven waves per SIMD)
__global__ __launch_bounds__(kKlThreads, 8) void kl_rows_kernel(
    const uint16_t* __restrict__ zc, const uint16_t* __restrict__ zp, int V,
    int64_t ld, float inv_tau, float* __restrict__ kl_out) {
  __shared__ KlState wst[kKlThreads / 64];
  __shared__ int whit[kKlThreads / 64];
  const int64_t row = blockIdx.x;
  const uint16_t* a = zc + row * ld;
  const uint16_t* b = zp + row * ld;
  const float l2t = kLog2e * inv_tau;
  const int wave = threadIdx.x >> 6;
  const bool lead = (threadIdx.x & 63) == 0;
  bool hit = false;
  float dref = row_reference<false>(a, b, V);
  KlState st = kl_row_pass<false>(a, b, V, l2t, inv_tau, dref, hit);
  if (lead) wst[wave] = st;
  __syncthreads();
  KlState t = merged_state(wst);
  // A second pass, always in masked mode (on finite data it does the plain
  // pass's arithmetic): when the state is not finite (masked tokens or other
  // non-finite data), and again, re-centred, when the result is a small
  // difference of large terms.  One copy of the masked pass, in a loop that
  // is not unrolled.
  bool again = !state_finite(t);
  if (again) {
    dref = row_reference<true>(a, b, V);
  } else if (t.s > 0.0f && amplified(t)) {
    again = true;
    dref = (float)((double)dref + (double)(t.u1 / t.s) / (double)inv_tau);
  }
  bool any_hit = false;
#pragma nounroll
  for (int k = 0; k < 2 && again; ++k) {
    __syncthreads();   // every thread has read wst and whit
    hit = false;
    st = kl_row_pass<true>(a, b, V, l2t, inv_tau, dref, hit);
    const bool wave_hit = __ballot(hit) != 0ull;
    if (lead) {
      wst[wave] = st;
      whit[wave] = wave_hit ? 1 : 0;
    }
    __syncthreads();
    t = merged_state(wst);
#pragma unroll
    for (int w = 0; w < kKlThreads / 64; ++w) any_hit = any_hit || whit[w] != 0;
    again = !any_hit && state_finite(t) && t.s > 0.0f && amplified(t);
    if (again) dref = (float)((double)dref + (double)(t.u1 / t.s) / (double)inv_tau);
  }
  if (threadIdx.x == 0) {
    const double s = t.s;
    const double x = ((double)t.u1 + (double)t.u3) / s;
    const double kl = any_hit ? (double)INFINITY : (double)t.u3 / s + (log1p(x) - x);
    kl_out[row] = (float)kl;
  }
}

// Mean of n per-row KL values in a fixed order (fp64), then the controller.
__global__ __launch_bounds__(1024) void kl_mean_kernel(const float* __restrict__ kl,
                                                       int n, float kl_budget,
                                                       float alpha_max,
                                                       float* __restrict__ q_alpha) {
  __shared__ double part[1024 / 64];
  double acc = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) acc += (double)kl[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int w = 0; w < 1024 / 64; ++w) tot += part[w];
    const double q = tot / (double)n;
    double alpha;
    if (isnan(q)) {
      alpha = NAN;
    } else if (q <= 0.0) {   // (q = +inf gives alpha = sqrt(0) = 0 below)
      alpha = alpha_max;
    } else {
      alpha = fmin((double)alpha_max, sqrt((double)kl_budget / q));
    }
    q_alpha[0] = (float)q;
    q_alpha[1] = (float)alpha;
  }
}

}  // namespace

hipError_t launch_kl(const uint16_t* zc, const uint16_t* zp, int n_tok,
                     int vocab, int64_t ld, float tau, float kl_budget,
                     float alpha_max, float* q_alpha, float* kl_tok,
                     hipStream_t s) {
  hipLaunchKernelGGL(kl_rows_kernel, dim3((unsigned)n_tok), dim3(kKlThreads), 0, s,
                     zc, zp, vocab, ld, 1.0f / tau, kl_tok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kl_mean_kernel, dim3(1), dim3(1024), 0, s, kl_tok, n_tok,
                     kl_budget, alpha_max, q_alpha);
  return hipGetLastError();
}

}  // namespace logra
