// logra_predicted_kl_sweep: the predicted KL at several step multipliers in
// one pass over the current logits z and the update direction delta, on gfx950.
//
// [LoGRA] (wispaper.ai summary of "LoGRA: Scaling LLM Reinforcement Learning
// with Low-Rank Gradient Sketches"), section PKL: the proposal is the current
// model moved along the update; at one common temperature its vocabulary
// distribution is compared with the current one, and the mean predicted KL
// grows as alpha^2 q(D).  Here the proposed logits z + alpha delta are formed
// in fp32 registers for every multiplier, never rounded to bf16, so the
// alpha^2 law holds on the inputs as given.
//
// With a = z/tau, dl = (delta - c)/tau, p = softmax(a) and w = e^(a - max):
//   KL(alpha) = log E_p[e^(alpha dl)] - alpha E_p[dl]
//             = g/s + log1p(x) - x,   x = (alpha u1 + g)/s,
//   s = sum w,  u1 = sum w dl,  g = sum w (e^(alpha dl) - 1 - alpha dl).
// The multiplier enters only through g, and
//   g(alpha) = sum_{n=2..8} alpha^n / n! * M_n + R(alpha),
//   M_n = sum w dl^n over the elements with amax |dl| <= 1 (amax = max |alpha|;
//         there the dropped tail of the series is below 1.1e-5 of
//         e^t - 1 - t, t = alpha dl),
//   R(alpha) = sum w (e^(alpha dl) - 1 - alpha dl) over the rare other
//         elements, evaluated exactly for each multiplier.
// The kernel carries u1, the M_n and the multipliers in units of u = amax dl
// (|u| <= 1 on the series path, so no power can overflow) and alpha / amax;
// the products alpha^n M_n are the same.
// c is a per-row reference, the mean of delta over the row's first min(V, 64)
// elements: adding alpha c to every proposed logit of a row leaves every
// KL(alpha) unchanged, and taking it out keeps a common offset of the
// direction out of the moments, where it would dominate them and cancel in
// the finalisation (and push every element off the series path).
// Masked tokens: a current logit of -inf is a token of probability zero, and
// it stays masked in every proposal whatever its direction entry (NaN and
// inf included).  The first pass over a row does not look for them (they
// leave some sum of the state non-finite); a row whose merged state is not
// finite is read a second time in masked mode, which skips those tokens and
// takes the direction reference from the others.  Rows of finite inputs pay
// one check.  The reference itself is checked the same way: a row whose KLs
// may be a small difference of large terms (the first 64 tokens missed an
// offset the rest of the row carries) is read again about the p-weighted
// mean of the direction, which its state already holds (sw_amplified).
// So an element costs the same ~20 VALU operations whatever the number of
// multipliers (dl itself is never formed: each element's u = amax dl comes
// from delta with one subtraction and one multiplication).  States merge by
// rescaling to the larger running max (shuffles inside a wave, LDS across
// the four waves of a row); rows are finalised in fp64 and a one-work-group
// kernel forms the weighted means in a fixed order.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"
#include "logra.h"

namespace logra {

namespace {

constexpr int kSwThreads = 256;
constexpr int kMoments = 7;       // M_2 .. M_8
constexpr float kSwLog2e = 1.4426950408889634f;

template <int NA>
struct SwState {
  float m;             // running max of a, in log2 units
  float s, u1;
  float M[kMoments];
  float r[NA];         // exact excess of the elements off the series
};

template <int NA>
__device__ __forceinline__ void sw_scale(SwState<NA>& st, float f) {
  st.s *= f;
  st.u1 *= f;
#pragma unroll
  for (int n = 0; n < kMoments; ++n) st.M[n] *= f;
#pragma unroll
  for (int i = 0; i < NA; ++i) st.r[i] *= f;
}

template <int NA>
__device__ __forceinline__ SwState<NA> sw_merge(SwState<NA> a, const SwState<NA>& b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return a;
  const float fa = a.m == -INFINITY ? 0.0f : exp2f(a.m - M);
  const float fb = b.m == -INFINITY ? 0.0f : exp2f(b.m - M);
  a.m = M;
  a.s = a.s * fa + b.s * fb;
  a.u1 = a.u1 * fa + b.u1 * fb;
#pragma unroll
  for (int n = 0; n < kMoments; ++n) a.M[n] = a.M[n] * fa + b.M[n] * fb;
#pragma unroll
  for (int i = 0; i < NA; ++i) a.r[i] = a.r[i] * fa + b.r[i] * fb;
  return a;
}

// e^t - 1 - t without cancellation: Taylor to t^7 for |t| <= 1/2 (relative
// truncation below 4e-6), exp otherwise.
__device__ __forceinline__ float sw_excess(float t) {
  float p = 1.0f / 5040.0f;
  p = fmaf(p, t, 1.0f / 720.0f);
  p = fmaf(p, t, 1.0f / 120.0f);
  p = fmaf(p, t, 1.0f / 24.0f);
  p = fmaf(p, t, 1.0f / 6.0f);
  p = fmaf(p, t, 0.5f);
  float g = t * t * p;
  if (fabsf(t) > 0.5f) g = expf(t) - 1.0f - t;
  return g;
}

struct Multipliers {
  float a[LOGRA_MAX_SWEEP];
};

// Adds n (<= 8) elements: z and dz are the logits and the direction.  The
// direction enters as u = dz su with su = max|alpha| / tau, so |u| <= 1 on
// the series path (its powers cannot overflow) and the multipliers are
// as = alpha / max|alpha| (alpha dz / tau = as u).  The weight exponent is
// z l2t - m in one fma (the running max is taken over z: l2t > 0 and
// rounding is monotonic, so max(z) l2t rounds to the max of the z l2t).
template <bool MASK, int NA>
__device__ __forceinline__ void sw_group(SwState<NA>& st, const float* z, const float* dz,
                                         int n, float l2t, float su, float thr,
                                         const Multipliers& as, float dref) {
  float zmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) zmax = fmaxf(zmax, e < n ? z[e] : -INFINITY);
  const float cmax = zmax * l2t;
  if (cmax > st.m) {
    sw_scale(st, st.m == -INFINITY ? 0.0f : exp2f(st.m - cmax));
    st.m = cmax;
  }
  const float nm = -st.m;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // MASK: a masked token (z = -inf) is skipped outright, its direction
    // entry unread
    if (e < n && (!MASK || z[e] != -INFINITY)) {
      const float w = exp2_normal(fmaf(z[e], l2t, nm));
      const float d = (dz[e] - dref) * su;
      st.s += w;
      float y = w * d;
      st.u1 += y;
      if (__builtin_expect(fabsf(d) <= thr, 1)) {
#pragma unroll
        for (int k = 0; k < kMoments; ++k) {
          y *= d;
          st.M[k] += y;
        }
      } else {
#pragma unroll
        for (int i = 0; i < NA; ++i) st.r[i] = fmaf(w, sw_excess(as.a[i] * d), st.r[i]);
      }
    }
  }
}

template <int NA>
__device__ __forceinline__ SwState<NA> sw_shfl_xor(const SwState<NA>& st, int off) {
  SwState<NA> o;
  o.m = __shfl_xor(st.m, off);
  o.s = __shfl_xor(st.s, off);
  o.u1 = __shfl_xor(st.u1, off);
#pragma unroll
  for (int n = 0; n < kMoments; ++n) o.M[n] = __shfl_xor(st.M[n], off);
#pragma unroll
  for (int i = 0; i < NA; ++i) o.r[i] = __shfl_xor(st.r[i], off);
  return o;
}

// Mean of delta over the first min(V, 64) elements of a row by a butterfly
// sum; every lane and wave of the row ends with the same bits (each level
// adds the same two partial sums, and fp32 addition is commutative).  MASK:
// over the unmasked tokens among them (0 when there is none).
template <bool MASK>
__device__ __forceinline__ float direction_reference(const uint16_t* zr, const uint16_t* dr,
                                                     int V) {
  const int lane = threadIdx.x & 63;
  const int nref = V < 64 ? V : 64;
  if constexpr (MASK) {
    const bool ok = lane < nref && bf16_to_f32(zr[lane]) != -INFINITY;
    float x = ok ? bf16_to_f32(dr[lane]) : 0.0f;
    float cnt = ok ? 1.0f : 0.0f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      x += __shfl_xor(x, off);
      cnt += __shfl_xor(cnt, off);
    }
    return cnt > 0.0f ? x / cnt : 0.0f;
  } else {
    float x = lane < nref ? bf16_to_f32(dr[lane]) : 0.0f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x / (float)nref;
  }
}

template <int NA>
__device__ __forceinline__ bool sw_finite(const SwState<NA>& t) {
  bool f = isfinite(t.s) && isfinite(t.u1);
#pragma unroll
  for (int n = 0; n < kMoments; ++n) f = f && isfinite(t.M[n]);
#pragma unroll
  for (int i = 0; i < NA; ++i) f = f && isfinite(t.r[i]);
  return f;
}

// One pass over a row with direction reference dref: this thread's
// elements, then the wave's butterfly (every lane ends with the wave's state).
template <bool MASK, int NA>
__device__ __forceinline__ SwState<NA> sw_row_pass(const uint16_t* zr, const uint16_t* dr, int V,
                                                   float l2t, float su, float thr,
                                                   const Multipliers& al, float dref) {
  SwState<NA> st;
  st.m = -INFINITY;
  st.s = 0.0f;
  st.u1 = 0.0f;
#pragma unroll
  for (int n = 0; n < kMoments; ++n) st.M[n] = 0.0f;
#pragma unroll
  for (int i = 0; i < NA; ++i) st.r[i] = 0.0f;

  // logits and direction are read once: non-temporal loads
  const int nfull = V >> 3;
  for (int c = threadIdx.x; c < nfull; c += kSwThreads) {
    const u32x4 va = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(zr + 8 * c));
    const u32x4 vb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dr + 8 * c));
    float zz[8], dd[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      zz[2 * p] = bf16_lo(va[p]);
      zz[2 * p + 1] = bf16_hi(va[p]);
      dd[2 * p] = bf16_lo(vb[p]);
      dd[2 * p + 1] = bf16_hi(vb[p]);
    }
    sw_group<MASK>(st, zz, dd, 8, l2t, su, thr, al, dref);
  }
  const int tail = V - 8 * nfull;
  if (tail > 0 && (int)threadIdx.x == nfull % kSwThreads) {
    float zz[8], dd[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      zz[e] = e < tail ? bf16_to_f32(zr[8 * nfull + e]) : 0.0f;
      dd[e] = e < tail ? bf16_to_f32(dr[8 * nfull + e]) : 0.0f;
    }
    sw_group<MASK>(st, zz, dd, tail, l2t, su, thr, al, dref);
  }
  // wave reduction (fixed butterfly)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) st = sw_merge(st, sw_shfl_xor(st, off));
  return st;
}

// A row is read once more, re-centred, when its KLs may have come out as a
// small difference of large terms.  With the reference near the p-weighted
// mean of the direction, g / s is about KL (both ~ alpha^2 Var_p(u) / 2 on
// small steps); an offset that the row's first 64 tokens do not share leaves
// E_p[u] far from 0 and the truncation and rounding of the sums enlarged by
// E_p[u^2] / Var_p(u).  The pass is repeated when that ratio may exceed 8:
// E_p[u]^2 > (7/8) E_p[u^2], taken as (u1/s)^2 > (7/8) M_2/s (M_2 holds
// the series elements, nearly all of them on small steps; when many are off
// the series this errs towards one more pass).  E_p[u] = u1 / s, so the next
// pass takes dref + u1 / (s su).
template <int NA>
__device__ __forceinline__ bool sw_amplified(const SwState<NA>& t) {
  const float e1 = t.u1 / t.s;
  return e1 * e1 > 0.875f * (t.M[0] / t.s);
}

// The four wave states merged in order; every thread that calls this gets
// the same bits, so choices made on the result are work-group uniform.
template <int NA>
__device__ __forceinline__ SwState<NA> sw_merged(const SwState<NA>* wst) {
  SwState<NA> t = wst[0];
#pragma unroll
  for (int w = 1; w < kSwThreads / 64; ++w) t = sw_merge(t, wst[w]);
  return t;
}

// One work-group per row: kl_out[i * n_tok + row] = KL_row(alpha_i).
template <int NA>
__global__ __launch_bounds__(kSwThreads, 8) void kl_sweep_rows_kernel(
    const uint16_t* __restrict__ z, const uint16_t* __restrict__ dz, int V, int64_t ld,
    int n_tok, int na, Multipliers al, float inv_tau, float su, float thr,
    float* __restrict__ kl_out) {
  __shared__ SwState<NA> wst[kSwThreads / 64];
  const int64_t row = blockIdx.x;
  const uint16_t* zr = z + row * ld;
  const uint16_t* dr = dz + row * ld;
  const float l2t = kSwLog2e * inv_tau;
  const int wave = threadIdx.x >> 6;
  const bool lead = (threadIdx.x & 63) == 0;
  float dref = direction_reference<false>(zr, dr, V);
  SwState<NA> st = sw_row_pass<false, NA>(zr, dr, V, l2t, su, thr, al, dref);
  if (lead) wst[wave] = st;
  __syncthreads();
  SwState<NA> t = sw_merged(wst);
  // A second pass, always in masked mode (on finite data it does the plain
  // pass's arithmetic): when the state is not finite (masked tokens or other
  // non-finite data), and again, re-centred, when the KLs may be a small
  // difference of large terms.  One copy of the masked pass, in a loop that
  // is not unrolled.
  bool again = !sw_finite(t);
  if (again) {
    dref = direction_reference<true>(zr, dr, V);
  } else if (t.s > 0.0f && sw_amplified(t)) {
    again = true;
    dref = (float)((double)dref + (double)(t.u1 / t.s) / (double)su);
  }
#pragma nounroll
  for (int k = 0; k < 2 && again; ++k) {
    __syncthreads();   // every thread has read wst
    st = sw_row_pass<true, NA>(zr, dr, V, l2t, su, thr, al, dref);
    if (lead) wst[wave] = st;
    __syncthreads();
    t = sw_merged(wst);
    again = k == 0 && sw_finite(t) && t.s > 0.0f && sw_amplified(t);
    if (again) dref = (float)((double)dref + (double)(t.u1 / t.s) / (double)su);
  }
  // then the multipliers' KLs (fp64)
  if (threadIdx.x == 0) {
    const double s = t.s;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (i < na) {
        const double a = al.a[i];   // alpha / max|alpha|: the moments are in units of u
        double g = t.r[i];
        double an = a * a, fact = 2.0;
#pragma unroll
        for (int n = 0; n < kMoments; ++n) {
          g += an / fact * (double)t.M[n];
          an *= a;
          fact *= (double)(n + 3);
        }
        const double x = (a * (double)t.u1 + g) / s;
        kl_out[(int64_t)i * n_tok + row] = (float)(g / s + (log1p(x) - x));
      }
    }
  }
}

// kl_mean[i] = sum_t w_t KL_t(alpha_i) / sum_t w_t in fp64, in a fixed order
// (equal weights when `weight` is null; a zero weight sum gives NaN).  A row
// of weight zero is left out whatever its KL: a masked position (padding
// with every logit -inf, say) may have none.
__global__ __launch_bounds__(1024) void kl_sweep_mean_kernel(const float* __restrict__ kl,
                                                             const float* __restrict__ weight,
                                                             int n, int na,
                                                             float* __restrict__ kl_mean) {
  __shared__ double part[2][1024 / 64];
  for (int i = 0; i < na; ++i) {
    const float* row = kl + (int64_t)i * n;
    double acc = 0.0, wacc = 0.0;
    for (int t = threadIdx.x; t < n; t += 1024) {
      const double w = weight ? (double)weight[t] : 1.0;
      if (w != 0.0) acc += w * (double)row[t];
      wacc += w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      acc += __shfl_xor(acc, off);
      wacc += __shfl_xor(wacc, off);
    }
    if ((threadIdx.x & 63) == 0) {
      part[0][threadIdx.x >> 6] = acc;
      part[1][threadIdx.x >> 6] = wacc;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double tot = 0.0, wtot = 0.0;
      for (int w = 0; w < 1024 / 64; ++w) {
        tot += part[0][w];
        wtot += part[1][w];
      }
      kl_mean[i] = wtot == 0.0 ? NAN : (float)(tot / wtot);
    }
    __syncthreads();
  }
}

template <int NA>
hipError_t launch_rows(const uint16_t* z, const uint16_t* dz, int n_tok, int vocab,
                       int64_t ld, int na, const Multipliers& al, float inv_tau, float su,
                       float thr, float* kl_tok, hipStream_t s) {
  hipLaunchKernelGGL((kl_sweep_rows_kernel<NA>), dim3((unsigned)n_tok), dim3(kSwThreads), 0,
                     s, z, dz, vocab, ld, n_tok, na, al, inv_tau, su, thr, kl_tok);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kl_sweep(const uint16_t* z, const uint16_t* dz, int n_tok, int vocab,
                           int64_t ld, const float* alphas, int n_alpha, float tau,
                           const float* weight, float* kl_mean, float* kl_tok,
                           hipStream_t s) {
  float amax = 0.0f;
  for (int i = 0; i < n_alpha; ++i) amax = fmaxf(amax, fabsf(alphas[i]));
  const float inv_tau = 1.0f / tau;
  // u = delta su with su = amax / tau, multipliers alpha / amax: the series
  // covers |u| <= 1 (amax |delta / tau| <= 1).  All multipliers zero: u =
  // delta / tau, every element on the series, every KL zero.
  Multipliers al{};
  float su = inv_tau, thr = INFINITY;
  if (amax > 0.0f) {
    su = (float)((double)amax / (double)tau);
    thr = 1.0f;
    for (int i = 0; i < n_alpha; ++i) al.a[i] = (float)((double)alphas[i] / (double)amax);
  }
  hipError_t e;
  if (n_alpha <= 1)
    e = launch_rows<1>(z, dz, n_tok, vocab, ld, n_alpha, al, inv_tau, su, thr, kl_tok, s);
  else if (n_alpha <= 2)
    e = launch_rows<2>(z, dz, n_tok, vocab, ld, n_alpha, al, inv_tau, su, thr, kl_tok, s);
  else if (n_alpha <= 4)
    e = launch_rows<4>(z, dz, n_tok, vocab, ld, n_alpha, al, inv_tau, su, thr, kl_tok, s);
  else
    e = launch_rows<8>(z, dz, n_tok, vocab, ld, n_alpha, al, inv_tau, su, thr, kl_tok, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kl_sweep_mean_kernel, dim3(1), dim3(1024), 0, s, kl_tok, weight, n_tok,
                     n_alpha, kl_mean);
  return hipGetLastError();
}

}  // namespace logra
