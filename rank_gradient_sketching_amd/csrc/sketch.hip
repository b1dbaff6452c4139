// logra_sketch_accumulate: S += dY^T (X A^T) for one microbatch, on gfx950.
//
// [LoGRA] (wispaper.ai summary of "LoGRA: Scaling LLM Reinforcement Learning
// with Low-Rank Gradient Sketches"), section Sketch: each microbatch's
// contribution to the d x r sketch S = G A^T is accumulated in fp32 by
// projecting the layer inputs first and only then multiplying with the
// backward derivatives, so the d x k gradient is never formed.
//
// Two kernels on the caller's stream:
//   project    P = c * X A^T (T x r).  One work-group per 32 tokens; its four
//              waves split k in 256-column chunks.  For the sign basis each
//              lane regenerates the sign bits of its A row in registers from
//              Philox (one block per row and chunk) and expands them to bf16
//              +-1 MFMA operands, so A never touches memory.  Products with
//              +-1 are exact; 32x32x16 bf16 MFMA accumulates in fp32; the
//              waves' partial sums meet in LDS in a fixed order.  P is written
//              transposed (r x T, tokens contiguous) as a hi/lo bf16 pair.
//   accumulate S += dY^T P.  A work-group owns 16*Q columns of d and a range
//              of 32-token steps.  Each lane loads an 8-token x Q-column block
//              of dY with row-contiguous loads and transposes it in registers
//              (v_perm_b32), giving K = token operands for 16x16x32 MFMA
//              against P_hi and P_lo.  Waves split the steps and are summed in
//              LDS in a fixed order; work-groups along T write partial tiles
//              and the last one to finish (device-scope counter) adds them to
//              S in split order, so S is bit-reproducible.
// The Gaussian basis is first written once per call as a bf16 r x k matrix in
// the workspace (Box-Muller per entry is too costly to repeat per token
// block) and the project kernel reads its operand tiles from there.
#include "common.hpp"
#include "internal.hpp"

namespace logra {

namespace {

constexpr int kProjWaves = 4;
constexpr int kAccWaves = 4;

// ------------------------------------------------------------------ project
template <int NB, bool GAUSS>
__global__ __launch_bounds__(256) void project_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, int T, int k, int r,
    uint64_t seed, uint64_t stream, float c, const uint16_t* __restrict__ Ab,
    int64_t lda, uint16_t* __restrict__ Phi, uint16_t* __restrict__ Plo,
    int64_t ldp, uint32_t* __restrict__ counters, int n_counters) {
  __shared__ float red[kProjWaves][32 * 33];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 31;  // A-operand row (token) and B-operand column (A row)
  const int h = lane >> 5;  // which half of each 256-column chunk this lane feeds
  const int t0 = blockIdx.x * 32;

  // The accumulate kernel that follows on the stream counts finished
  // work-groups per column group; reset its counters here.
  if (blockIdx.x == 0) {
    for (int i = tid; i < n_counters; i += 256) counters[i] = 0u;
  }

  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[nb][v] = 0.0f;
  }

  const int t = t0 + m;
  const bool trow = t < T;
  const uint16_t* xrow = X + (int64_t)(trow ? t : 0) * ldx;
  const int n_chunks = (k + 255) >> 8;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  for (int ch = wave; ch < n_chunks; ch += kProjWaves) {
    // K assignment: in step s, lane half h carries columns
    // 256 ch + 128 h + 8 s + (0..7).
    const int cbase = ch * 256 + h * 128;
    u32x4 xv[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      xv[s] = trow ? load_bf16x8(xrow, cbase + 8 * s, k) : zero4;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int i = nb * 32 + m;  // row of A feeding B-operand column m
      if (GAUSS) {
        const uint16_t* arow = Ab + (int64_t)i * lda + cbase;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const u32x4 b = *reinterpret_cast<const u32x4*>(arow + 8 * s);
          acc[nb] = mfma32(xv[s], b, acc[nb]);
        }
      } else {
        uint64_t w0 = 0, w1 = 0;
        if (i < r) {
          const Words4 blk = sign_block(seed, stream, (uint64_t)ch, (uint64_t)i);
          w0 = h ? blk.w[2] : blk.w[0];
          w1 = h ? blk.w[3] : blk.w[1];
        }
        const bool live = i < r;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const uint64_t w = s < 8 ? w0 : w1;
          const uint32_t byte = (uint32_t)(w >> (8 * (s & 7))) & 0xFFu;
          const u32x4 b = live ? signs_to_bf16x8(byte) : zero4;
          acc[nb] = mfma32(xv[s], b, acc[nb]);
        }
      }
    }
  }

  // Sum the four waves' partial P in a fixed order and write P^T as hi/lo.
  const int n_out = tid & 31;   // A row within the block
  const int tg = tid >> 5;      // tokens 4 tg .. 4 tg + 3
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 8 * (v >> 2) + 4 * h + (v & 3);
      red[wave][row * 33 + m] = acc[nb][v];
    }
    __syncthreads();
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = (4 * tg + u) * 33 + n_out;
      float p = ((red[0][idx] + red[1][idx]) + red[2][idx]) + red[3][idx];
      split_bf16(p * c, hi[u], lo[u]);
    }
    const int64_t off = (int64_t)(nb * 32 + n_out) * ldp + t0 + 4 * tg;
    u32x2 vh, vl;
    vh[0] = (uint32_t)hi[0] | ((uint32_t)hi[1] << 16);
    vh[1] = (uint32_t)hi[2] | ((uint32_t)hi[3] << 16);
    vl[0] = (uint32_t)lo[0] | ((uint32_t)lo[1] << 16);
    vl[1] = (uint32_t)lo[2] | ((uint32_t)lo[3] << 16);
    *reinterpret_cast<u32x2*>(Phi + off) = vh;
    *reinterpret_cast<u32x2*>(Plo + off) = vl;
    __syncthreads();
  }
}

// Writes the Gaussian basis as bf16 rows of length lda (rows >= r and columns
// >= k are zero), one thread per (row, 4-column group).
__global__ __launch_bounds__(256) void gauss_basis_kernel(
    uint64_t seed, uint64_t stream, int r, int k, int rows, int64_t lda,
    float cr, uint16_t* __restrict__ Ab) {
  const int64_t groups = lda >> 2;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)rows * groups) return;
  const int64_t row = id / groups;
  const int64_t q = id % groups;
  uint16_t v[4] = {0, 0, 0, 0};
  if (row < r && 4 * q < k) {
    gaussian_entries_bf16(seed, stream, (uint64_t)q, (uint64_t)row, cr, v);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if (4 * q + a >= k) v[a] = 0;
    }
  }
  u32x2 w;
  w[0] = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
  w[1] = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
  *reinterpret_cast<u32x2*>(Ab + row * lda + 4 * q) = w;
}

// --------------------------------------------------------------- accumulate
template <int Q>
struct DyBlock;
template <>
struct DyBlock<8> {
  u32x4 v;
};
template <>
struct DyBlock<4> {
  u32x2 v;
};
template <>
struct DyBlock<2> {
  uint32_t v;
};

// Q bf16 of one dY row starting at column `col` (zeros past `ncols`).
template <int Q>
__device__ __forceinline__ void load_dy(const uint16_t* row, int col, int ncols,
                                        uint32_t out[Q / 2]) {
  if (col + Q <= ncols) {
    if constexpr (Q == 8) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(row + col);
#pragma unroll
      for (int p = 0; p < 4; ++p) out[p] = v[p];
    } else if constexpr (Q == 4) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(row + col);
      out[0] = v[0];
      out[1] = v[1];
    } else {
      out[0] = *reinterpret_cast<const uint32_t*>(row + col);
    }
    return;
  }
#pragma unroll
  for (int p = 0; p < Q / 2; ++p) out[p] = 0u;
#pragma unroll
  for (int e = 0; e < Q; ++e) {
    if (col + e < ncols) {
      const uint32_t hv = row[col + e];
      out[e >> 1] |= (e & 1) ? (hv << 16) : hv;
    }
  }
}

template <int Q, int NB16>
__global__ __launch_bounds__(256) void accumulate_kernel(
    const uint16_t* __restrict__ dY, int64_t ldd, int T, int d, int r,
    const uint16_t* __restrict__ Phi, const uint16_t* __restrict__ Plo,
    int64_t ldp, int steps_total, int steps_per_split, int n_split,
    float* __restrict__ S, float* __restrict__ part, int64_t d_pad,
    uint32_t* __restrict__ counters) {
  constexpr int RP = 16 * NB16;   // padded r handled here
  constexpr int DC = 16 * Q;      // d columns per work-group
  constexpr int NREG = Q * NB16 * 4;
  __shared__ float red[NREG * 64];
  __shared__ int is_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 15;   // A-operand row group (d) and B-operand column (r)
  const int g4 = lane >> 4;  // which 8 tokens of the 32-token step
  const int dg = blockIdx.x;
  const int sp = blockIdx.y;
  const int dc0 = dg * DC;
  const int col = dc0 + Q * m;
  const int s_begin = sp * steps_per_split;
  const int s_end = min(steps_total, s_begin + steps_per_split);

  f32x4 acc[Q][NB16];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
#pragma unroll
    for (int nb = 0; nb < NB16; ++nb) acc[q][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int st = s_begin + wave; st < s_end; st += kAccWaves) {
    const int tb = st * 32 + 8 * g4;
    uint32_t R[8][Q / 2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = tb + e;
      if (t < T) {
        load_dy<Q>(dY + (int64_t)t * ldd, col, d, R[e]);
      } else {
#pragma unroll
        for (int p = 0; p < Q / 2; ++p) R[e][p] = 0u;
      }
    }
    u32x4 bh[NB16], bl[NB16];
#pragma unroll
    for (int nb = 0; nb < NB16; ++nb) {
      const int64_t off = (int64_t)(16 * nb + m) * ldp + tb;
      bh[nb] = *reinterpret_cast<const u32x4*>(Phi + off);
      bl[nb] = *reinterpret_cast<const u32x4*>(Plo + off);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      // K assignment: lane group g4, element e <-> token tb + e.
      u32x4 a;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = __builtin_amdgcn_perm(R[2 * u + 1][q >> 1], R[2 * u][q >> 1],
                                     (q & 1) ? 0x07060302u : 0x05040100u);
      }
#pragma unroll
      for (int nb = 0; nb < NB16; ++nb) {
        acc[q][nb] = mfma16(a, bh[nb], acc[q][nb]);
        acc[q][nb] = mfma16(a, bl[nb], acc[q][nb]);
      }
    }
  }

  // Fixed-order sum of the four waves: ((w0 + w1) + (w2 + w3)).
  auto store_lds = [&]() {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int nb = 0; nb < NB16; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          red[((q * NB16 + nb) * 4 + v) * 64 + lane] = acc[q][nb][v];
  };
  auto add_lds = [&]() {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int nb = 0; nb < NB16; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[q][nb][v] += red[((q * NB16 + nb) * 4 + v) * 64 + lane];
  };
  if (wave == 1) store_lds();
  __syncthreads();
  if (wave == 0) add_lds();
  __syncthreads();
  if (wave == 3) store_lds();
  __syncthreads();
  if (wave == 2) add_lds();
  __syncthreads();
  if (wave == 2) store_lds();
  __syncthreads();
  if (wave == 0) add_lds();

  // Wave 0 lane (n = lane % 16, g = lane / 16) holds, for every (q, nb, v),
  // the value of d row dc0 + Q (4 g + v) + q, r column 16 nb + n.
  if (wave == 0) {
    const int n = lane & 15;
    const int g = lane >> 4;
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int nb = 0; nb < NB16; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int drow = dc0 + Q * (4 * g + v) + q;
          const int rc = 16 * nb + n;
          if (n_split == 1) {
            if (drow < d && rc < r) S[(int64_t)drow * r + rc] += acc[q][nb][v];
          } else {
            part[((int64_t)sp * d_pad + drow) * RP + rc] = acc[q][nb][v];
          }
        }
  }
  if (n_split == 1) return;

  // Last work-group of this column group adds the partial tiles to S.
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&counters[dg], 1u);
    is_last = (prev == (uint32_t)(n_split - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int idx = tid; idx < DC * RP; idx += 256) {
    const int drow = dc0 + idx / RP;
    const int rc = idx % RP;
    if (drow >= d || rc >= r) continue;
    const float* pp = part + (int64_t)drow * RP + rc;
    float sum = pp[0];
    for (int s = 1; s < n_split; ++s) sum += pp[(int64_t)s * d_pad * RP];
    S[(int64_t)drow * r + rc] += sum;
  }
  if (tid == 0) counters[dg] = 0u;
}

template <int NB>
hipError_t launch_project(const SketchPlan& p, const uint16_t* X, int64_t ldx,
                          int T, int k, int r, uint64_t seed, uint64_t stream,
                          bool gauss, float c, const uint16_t* Ab,
                          uint16_t* Phi, uint16_t* Plo, uint32_t* cnt,
                          hipStream_t s) {
  const dim3 grid((unsigned)(p.t_pad / 32));
  const int n_cnt = p.n_split > 1 ? p.n_dgroups : 0;
  if (gauss) {
    hipLaunchKernelGGL((project_kernel<NB, true>), grid, dim3(256), 0, s, X, ldx,
                       T, k, r, seed, stream, 1.0f, Ab, p.k_pad, Phi, Plo,
                       p.t_pad, cnt, n_cnt);
  } else {
    hipLaunchKernelGGL((project_kernel<NB, false>), grid, dim3(256), 0, s, X,
                       ldx, T, k, r, seed, stream, c, Ab, p.k_pad, Phi, Plo,
                       p.t_pad, cnt, n_cnt);
  }
  return hipGetLastError();
}

template <int Q, int NB16>
hipError_t launch_accumulate(const SketchPlan& p, const uint16_t* dY,
                             int64_t ldd, int T, int d, int r,
                             const uint16_t* Phi, const uint16_t* Plo, float* S,
                             float* part, uint32_t* cnt, hipStream_t s) {
  const dim3 grid((unsigned)p.n_dgroups, (unsigned)p.n_split);
  hipLaunchKernelGGL((accumulate_kernel<Q, NB16>), grid, dim3(256), 0, s, dY,
                     ldd, T, d, r, Phi, Plo, p.t_pad, p.steps,
                     p.steps_per_split, p.n_split, S, part, p.d_pad, cnt);
  return hipGetLastError();
}

}  // namespace

bool make_sketch_plan(int64_t T, int64_t d, int64_t k, int r, SketchPlan* p) {
  if (T < 0 || d < 1 || k < 1 || r < 1 || r > 256) return false;
  if (T >= (int64_t(1) << 31) || d >= (int64_t(1) << 31) ||
      k >= (int64_t(1) << 31))
    return false;
  SketchPlan q{};
  q.rp = r <= 16 ? 16 : r <= 32 ? 32 : r <= 64 ? 64 : r <= 128 ? 128 : 256;
  q.p_rows = q.rp < 32 ? 32 : q.rp;
  q.nb32 = q.p_rows / 32;
  q.q_cols = q.rp <= 64 ? 8 : q.rp == 128 ? 4 : 2;
  q.t_pad = round_up(T > 0 ? T : 1, 32);
  q.k_pad = round_up(k, 256);
  q.steps = (int)(q.t_pad / 32);
  const int dc = 16 * q.q_cols;
  q.n_dgroups = (int)((d + dc - 1) / dc);
  // Enough work-groups to cover the chip (256 CUs) while each wave keeps at
  // least two 32-token steps.
  const int want = (256 + q.n_dgroups - 1) / q.n_dgroups;
  const int max_split = q.steps / (2 * kAccWaves) > 0 ? q.steps / (2 * kAccWaves) : 1;
  int n_split = want < max_split ? want : max_split;
  if (n_split < 1) n_split = 1;
  q.steps_per_split = (q.steps + n_split - 1) / n_split;
  q.n_split = (q.steps + q.steps_per_split - 1) / q.steps_per_split;
  q.d_pad = (int64_t)q.n_dgroups * dc;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  const size_t p_bytes = (size_t)q.p_rows * (size_t)q.t_pad * 2;
  q.off_phi = take(p_bytes);
  q.off_plo = take(p_bytes);
  q.off_part = take(q.n_split > 1 ? (size_t)q.n_split * q.d_pad * q.rp * 4 : 0);
  q.off_cnt = take((size_t)q.n_dgroups * 4);
  q.off_gauss = take((size_t)q.p_rows * (size_t)q.k_pad * 2);
  q.total = off;
  *p = q;
  return true;
}

hipError_t launch_sketch(const SketchPlan& p, const uint16_t* X, int64_t ldx,
                         const uint16_t* dY, int64_t ldd, int T, int d, int k,
                         int r, uint64_t seed, uint64_t stream, int kind,
                         float* S, char* ws, hipStream_t s) {
  uint16_t* Phi = reinterpret_cast<uint16_t*>(ws + p.off_phi);
  uint16_t* Plo = reinterpret_cast<uint16_t*>(ws + p.off_plo);
  float* part = reinterpret_cast<float*>(ws + p.off_part);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + p.off_cnt);
  uint16_t* Ab = reinterpret_cast<uint16_t*>(ws + p.off_gauss);
  const bool gauss = kind == 1;
  const float c = sign_scale(r);
  hipError_t e = hipSuccess;
  if (gauss) {
    const int64_t threads = (int64_t)p.p_rows * (p.k_pad >> 2);
    hipLaunchKernelGGL(gauss_basis_kernel, dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, seed, stream, r, k, p.p_rows, p.k_pad, c,
                       Ab);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (p.nb32) {
    case 1: e = launch_project<1>(p, X, ldx, T, k, r, seed, stream, gauss, c, Ab, Phi, Plo, cnt, s); break;
    case 2: e = launch_project<2>(p, X, ldx, T, k, r, seed, stream, gauss, c, Ab, Phi, Plo, cnt, s); break;
    case 4: e = launch_project<4>(p, X, ldx, T, k, r, seed, stream, gauss, c, Ab, Phi, Plo, cnt, s); break;
    default: e = launch_project<8>(p, X, ldx, T, k, r, seed, stream, gauss, c, Ab, Phi, Plo, cnt, s); break;
  }
  if (e != hipSuccess) return e;
  switch (p.rp) {
    case 16: return launch_accumulate<8, 1>(p, dY, ldd, T, d, r, Phi, Plo, S, part, cnt, s);
    case 32: return launch_accumulate<8, 2>(p, dY, ldd, T, d, r, Phi, Plo, S, part, cnt, s);
    case 64: return launch_accumulate<8, 4>(p, dY, ldd, T, d, r, Phi, Plo, S, part, cnt, s);
    case 128: return launch_accumulate<4, 8>(p, dY, ldd, T, d, r, Phi, Plo, S, part, cnt, s);
    default: return launch_accumulate<2, 16>(p, dY, ldd, T, d, r, Phi, Plo, S, part, cnt, s);
  }
}

}  // namespace logra
