// logra_merge: W <- RNE_bf16(W - alpha * eta * S A) in place, on gfx950.
//
// [LoGRA] (wispaper.ai summary of "LoGRA: Scaling LLM Reinforcement Learning
// with Low-Rank Gradient Sketches"), section Sketch: the update is
// W <- W - alpha eta U A with U = S in the basic SGD variant, merged straight
// into the weights with no adapter branch; section Sync: the rollout engine
// applies the same merge after rebuilding A from the seed.
//
// One work-group owns 256 rows x 256 columns of W (one sign block wide); its
// four waves own 64 rows each.  Columns are processed in four passes of 64:
//   1. the pass's slice of A (r x 64) is regenerated into LDS as bf16,
//      transposed (column-major, r contiguous) - signs from registers holding
//      the Philox block of two A rows per thread, or Gaussian entries;
//   2. 16x16x32 bf16 MFMA with M = W columns, N = W rows, K = r computes the
//      slice of S A; S enters as a hi/lo bf16 pair, so the product keeps about
//      16 bits of S;
//   3. the lane owning 16 contiguous columns of one row loads them (two
//      16-byte loads issued before the MFMAs), subtracts the scaled product in
//      fp32 and rounds once to bf16 (v_cvt_pk_bf16_f32, ties to even).
// The M -> column map (m / 4) * 16 + 4 t + m % 4 makes each lane's 16
// accumulator values land on 16 consecutive columns of one row.
#include "common.hpp"
#include "internal.hpp"

namespace logra {

namespace {

constexpr int kMergeRows = 256;
constexpr int kMergeCols = 256;
constexpr int kPassCols = 64;

template <int NKS, bool GAUSS, bool MASKED>
__global__ __launch_bounds__(256) void merge_kernel(
    uint16_t* __restrict__ W, int64_t ldw, const float* __restrict__ S, int d,
    int k, int r, uint64_t seed, uint64_t stream, float scale, float cr) {
  constexpr int RP = 32 * NKS;    // r padded to whole K steps
  constexpr int LDA = RP + 8;     // bf16 per LDS column (+16 B against conflicts)
  constexpr bool kDouble = NKS <= 4;  // two A slices fit in 64 KB of LDS
  __shared__ uint16_t At[(kDouble ? 2 : 1) * kPassCols * LDA];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 15;   // A-operand row (column slot) and B/D column (row)
  const int g = lane >> 4;   // K group for operands, row group for D
  // flat grid: column block fastest, so neighbouring work-groups share rows
  const int n_cb = (k + kMergeCols - 1) / kMergeCols;
  const int cb = (int)(blockIdx.x % (unsigned)n_cb);
  const int rblk = (int)(blockIdx.x / (unsigned)n_cb);
  const int col0 = cb * kMergeCols;
  const int row0 = rblk * kMergeRows + wave * 64;
  const int n_pass = min(kMergeCols / kPassCols, (k - col0 + kPassCols - 1) / kPassCols);

  // S operands: rows row0 + 16 nt + m, K = r columns 32 ks + 8 g + (0..7),
  // as hi/lo bf16.  They do not depend on the column pass, so for small r
  // they stay in registers; for large r they are rebuilt per pass (L2 hits).
  constexpr bool kHoistS = NKS <= 2;
  // rows of this wave all inside d and r a multiple of 32: plain float4 loads
  const bool s_fast = !MASKED;
  auto s_operands = [&](int nt, int ks, u32x4& hi, u32x4& lo) {
    const int row = row0 + 16 * nt + m;
    float v[8];
    if (s_fast) {
      const f32x4* sp = reinterpret_cast<const f32x4*>(S + (int64_t)row * r + 32 * ks + 8 * g);
      const f32x4 a = sp[0], b = sp[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = a[e];
        v[4 + e] = b[e];
      }
    } else {
      const int rr = row < d ? row : d - 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int rc = 32 * ks + 8 * g + e;
        const float x = S[(int64_t)rr * r + (rc < r ? rc : r - 1)];
        v[e] = (row < d && rc < r) ? x : 0.0f;
      }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint16_t h0, l0, h1, l1;
      split_bf16(v[2 * p], h0, l0);
      split_bf16(v[2 * p + 1], h1, l1);
      hi[p] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      lo[p] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
  };
  u32x4 sh[4][kHoistS ? NKS : 1], sl[4][kHoistS ? NKS : 1];
  if constexpr (kHoistS) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) s_operands(nt, ks, sh[nt][ks], sl[nt][ks]);
  }

  // Sign basis: thread tid < RP / 2 keeps the Philox blocks of A rows
  // 2 tid and 2 tid + 1 for this 256-column block.
  uint64_t sw0[4] = {0, 0, 0, 0}, sw1[4] = {0, 0, 0, 0};
  const int ra = 2 * tid, rb = 2 * tid + 1;
  if (!GAUSS && tid < RP / 2) {
    if (ra < r) {
      const Words4 b = sign_block(seed, stream, (uint64_t)cb, (uint64_t)ra);
#pragma unroll
      for (int q = 0; q < 4; ++q) sw0[q] = b.w[q];
    }
    if (rb < r) {
      const Words4 b = sign_block(seed, stream, (uint64_t)cb, (uint64_t)rb);
#pragma unroll
      for (int q = 0; q < 4; ++q) sw1[q] = b.w[q];
    }
  }

  // A slice of pass p into LDS: buf[col * LDA + i] = A[i][col0 + 64 p + col].
  auto build_A = [&](int pass, uint16_t* buf) {
    const int c0 = col0 + pass * kPassCols;
    if (GAUSS) {
      for (int job = tid; job < RP * (kPassCols / 4); job += 256) {
        const int i = job / (kPassCols / 4);
        const int cc = 4 * (job % (kPassCols / 4));
        uint16_t v[4] = {0, 0, 0, 0};
        if (i < r && c0 + cc < k) {
          gaussian_entries_bf16(seed, stream, (uint64_t)((c0 + cc) >> 2),
                                (uint64_t)i, cr, v);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) buf[(cc + a) * LDA + i] = v[a];
      }
    } else if (tid < RP / 2) {
      // word `pass` of each block holds columns 64 pass .. 64 pass + 63
      const uint64_t wa = pass == 0 ? sw0[0] : pass == 1 ? sw0[1] : pass == 2 ? sw0[2] : sw0[3];
      const uint64_t wb = pass == 0 ? sw1[0] : pass == 1 ? sw1[1] : pass == 2 ? sw1[2] : sw1[3];
      const uint32_t one = 0x3F80u, neg = 0xBF80u;
      uint32_t* b32 = reinterpret_cast<uint32_t*>(buf);
#pragma unroll 8
      for (int cc = 0; cc < kPassCols; ++cc) {
        const uint32_t lo = ra < r ? (((wa >> cc) & 1u) ? neg : one) : 0u;
        const uint32_t hi = rb < r ? (((wb >> cc) & 1u) ? neg : one) : 0u;
        b32[(cc * LDA) / 2 + tid] = lo | (hi << 16);
      }
    }
  };

  // This lane's W elements of pass p: rows row0 + 16 nt + m, columns
  // col0 + 64 p + 16 g + (0..15).  Rows past d are read from row d - 1 and
  // never stored; columns past k read as zero.
  auto load_W = [&](int pass, u32x4 wv[4][2]) {
    const int c0 = col0 + pass * kPassCols;
    const int wc = c0 + 16 * g;
    if (!MASKED) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint16_t* wr = W + (int64_t)(row0 + 16 * nt + m) * ldw;
        wv[nt][0] = load_bf16x8(wr, wc);
        wv[nt][1] = load_bf16x8(wr, wc + 8);
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int row = min(row0 + 16 * nt + m, d - 1);
        const uint16_t* wr = W + (int64_t)row * ldw;
        wv[nt][0] = load_bf16x8_masked(wr, wc, k);
        wv[nt][1] = load_bf16x8_masked(wr, wc + 8, k);
      }
    }
  };

  uint16_t* buf0 = At;
  uint16_t* buf1 = At + (kDouble ? kPassCols * LDA : 0);

  // One column pass: multiply the A slice, update the W elements loaded one
  // pass earlier (wcur) and, before that, start the loads of the next pass
  // (wnxt) so they overlap this pass's work.
  auto do_pass = [&](int pass, u32x4 (&wcur)[4][2], u32x4 (&wnxt)[4][2]) {
    if (!kDouble && pass > 0) {
      __syncthreads();          // every wave is done reading the previous slice
      build_A(pass, buf0);
    }
    __syncthreads();            // slice `pass` is complete
    if (pass + 1 < n_pass) {
      load_W(pass + 1, wnxt);
      __builtin_amdgcn_sched_barrier(0);
      if (kDouble) build_A(pass + 1, (pass & 1) ? buf0 : buf1);
    }
    const uint16_t* cur_buf = (kDouble && (pass & 1)) ? buf1 : buf0;

    // MFMA: acc[t][nt] rows m' = 4 g' + v map to columns c0 + 16 g' + 4 t + v.
    f32x4 acc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 bh[4], bl[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if constexpr (kHoistS) {
          bh[nt] = sh[nt][ks];
          bl[nt] = sl[nt][ks];
        } else {
          s_operands(nt, ks, bh[nt], bl[nt]);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int cc = (m >> 2) * 16 + 4 * t + (m & 3);
        const u32x4 a =
            *reinterpret_cast<const u32x4*>(&cur_buf[cc * LDA + 32 * ks + 8 * g]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          acc[t][nt] = mfma16(a, bh[nt], acc[t][nt]);
          acc[t][nt] = mfma16(a, bl[nt], acc[t][nt]);
        }
      }
    }

    // Update and store.
    const int wc = col0 + pass * kPassCols + 16 * g;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int row = row0 + 16 * nt + m;
      u32x4 out[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          // element e = 8 hh + 2 p (+1) of the lane's 16 columns = 4 t + v
          const int e0 = 8 * hh + 2 * p;
          const int e1 = e0 + 1;
          const float w0 = bf16_lo(wcur[nt][hh][p]);
          const float w1 = bf16_hi(wcur[nt][hh][p]);
          const float n0 = w0 - scale * acc[e0 >> 2][nt][e0 & 3];
          const float n1 = w1 - scale * acc[e1 >> 2][nt][e1 & 3];
          out[hh][p] = pack_bf16x2(n0, n1);
        }
      }
      if (!MASKED || row < d) {
        uint16_t* wr = W + (int64_t)row * ldw;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int cbeg = wc + 8 * hh;
          if (!MASKED || cbeg + 8 <= k) {
            *reinterpret_cast<u32x4*>(wr + cbeg) = out[hh];
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (cbeg + e < k) {
                const uint32_t dw = out[hh][e >> 1];
                wr[cbeg + e] = (uint16_t)((e & 1) ? (dw >> 16) : (dw & 0xFFFFu));
              }
            }
          }
        }
      }
    }
  };

  u32x4 wa[4][2], wb[4][2];
  build_A(0, buf0);
  load_W(0, wa);
  do_pass(0, wa, wb);
  if (n_pass > 1) do_pass(1, wb, wa);
  if (n_pass > 2) do_pass(2, wa, wb);
  if (n_pass > 3) do_pass(3, wb, wa);
}

template <int NKS, bool MASKED>
void launch_merge_m(uint16_t* W, int64_t ldw, const float* S, int d, int k, int r,
                    uint64_t seed, uint64_t stream, bool gauss, float scale,
                    float cr, hipStream_t s, dim3 grid) {
  if (gauss) {
    hipLaunchKernelGGL((merge_kernel<NKS, true, MASKED>), grid, dim3(256), 0, s, W,
                       ldw, S, d, k, r, seed, stream, scale, cr);
  } else {
    hipLaunchKernelGGL((merge_kernel<NKS, false, MASKED>), grid, dim3(256), 0, s, W,
                       ldw, S, d, k, r, seed, stream, scale, cr);
  }
}

template <int NKS>
hipError_t launch_merge_t(uint16_t* W, int64_t ldw, const float* S, int d, int k,
                          int r, uint64_t seed, uint64_t stream, bool gauss,
                          float scale, float cr, hipStream_t s) {
  const int64_t blocks = (int64_t)((k + kMergeCols - 1) / kMergeCols) *
                         ((d + kMergeRows - 1) / kMergeRows);
  const dim3 grid((unsigned)blocks);
  // unmasked when every tile is interior and S rows are whole K steps
  const bool masked = (d % kMergeRows) != 0 || (k % kMergeCols) != 0 || (r % 32) != 0;
  if (masked) launch_merge_m<NKS, true>(W, ldw, S, d, k, r, seed, stream, gauss, scale, cr, s, grid);
  else launch_merge_m<NKS, false>(W, ldw, S, d, k, r, seed, stream, gauss, scale, cr, s, grid);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(uint16_t* W, int64_t ldw, const float* S, int d, int k,
                        int r, uint64_t seed, uint64_t stream, int kind,
                        float alpha, float eta, hipStream_t s) {
  const bool gauss = kind == 1;
  const float cr = sign_scale(r);
  const float step = alpha * eta;             // fp32 product, as documented
  const float scale = gauss ? step : step * cr;
  const int nks = (r + 31) / 32;
  switch (nks <= 1 ? 1 : nks <= 2 ? 2 : nks <= 4 ? 4 : 8) {
    case 1: return launch_merge_t<1>(W, ldw, S, d, k, r, seed, stream, gauss, scale, cr, s);
    case 2: return launch_merge_t<2>(W, ldw, S, d, k, r, seed, stream, gauss, scale, cr, s);
    case 4: return launch_merge_t<4>(W, ldw, S, d, k, r, seed, stream, gauss, scale, cr, s);
    default: return launch_merge_t<8>(W, ldw, S, d, k, r, seed, stream, gauss, scale, cr, s);
  }
}

}  // namespace logra
