// logra_merge: W <- RNE_bf16(W - alpha * eta * S A) in place, on gfx950.
//
// [LoGRA] (wispaper.ai summary of "LoGRA: Scaling LLM Reinforcement Learning
// with Low-Rank Gradient Sketches"), section Sketch: the update is
// W <- W - alpha eta U A with U = S in the basic SGD variant, merged straight
// into the weights with no adapter branch; section Sync: the rollout engine
// applies the same merge after rebuilding A from the seed.
//
// One work-group owns a block of rows x 256 columns of W (one sign block
// wide) and each of its waves 16 or 32 of those rows (the shapes are chosen
// per rank and basis below).  Columns are processed in four passes of 64:
//   1. the pass's slice of A (r x 64) is regenerated into LDS as bf16,
//      transposed (column-major, r contiguous) by all threads - signs from
//      the Philox words of the block's A rows (drawn once per work-group and
//      parked in LDS), or Gaussian entries;
//   2. 16x16x32 bf16 MFMA with M = W columns, N = W rows, K = r computes the
//      slice of S A; S enters as a hi/lo bf16 pair, so the product keeps about
//      16 bits of S;
//   3. the scaled product is subtracted from W in fp32 and rounded once to
//      bf16 (v_cvt_pk_bf16_f32, ties to even).
// The M -> column map (m / 4) * 16 + 4 t + m % 4 makes each lane's 16
// accumulator values land on 16 consecutive columns of one row.
// Interior tiles of 16-row waves with the sign basis (r <= 64) move W in
// whole 128-byte lines:
// each load and store instruction covers 8 rows x 128 B (8 lanes per row),
// non-temporal both ways, and the products reach that layout through a
// per-wave fp32 stage in LDS.  In the MFMA layout each instruction touched 16
// rows x 64 B (half lines); W's read-modify-write alone measured 17.9 us that
// way and 12.7 us coalesced and non-temporal (d = k = 4096, the rate of a
// device copy).  Other tiles load W in the MFMA layout and store whole lines
// through a bf16 stage.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace logra {

namespace {

constexpr int kMergeCols = 256;
constexpr int kPassCols = 64;

// The weights of a launch as its first kernel argument.  MergeOne: the one
// weight of logra_merge (the launch arguments stay as small as separate
// parameters; a launch's cost was measured to grow with its argument bytes).
// MergeTable: the weights of logra_merge_many; weight i owns the tasks
// t_off[i] .. t_off[i + 1] - 1, its row blocks x column blocks (column block
// fastest).  All share the rank, the basis kind and the step size.
struct MergeOne {
  uint16_t* W;
  int64_t ldw;
  const float* S;
  int d;
  int k;
  uint64_t seed;
  uint64_t stream;
};
struct MergeTable {
  int n;
  int t_off[kMaxMerge + 1];
  uint16_t* W[kMaxMerge];
  int64_t ldw[kMaxMerge];
  const float* S[kMaxMerge];
  int d[kMaxMerge];
  int k[kMaxMerge];
  uint64_t seed[kMaxMerge];
  uint64_t stream[kMaxMerge];
};

// The weight of task `task` and the task's index within the weight (table
// entries by compares and selects on constant indices).
struct MergeSel {
  MergeOne w;
  int local;
};
__device__ __forceinline__ MergeSel select_weight(const MergeOne& t, int task) {
  return MergeSel{t, task};
}
// (Each later weight that the task reaches overrides the fields: compares,
// not a variable index, which would copy the table to scratch memory.)
__device__ __forceinline__ MergeSel select_weight(const MergeTable& t, int task) {
  MergeSel q{MergeOne{t.W[0], t.ldw[0], t.S[0], t.d[0], t.k[0], t.seed[0], t.stream[0]},
             task - t.t_off[0]};
#pragma unroll
  for (int i = 1; i < kMaxMerge; ++i) {
    if (i < t.n && task >= t.t_off[i]) {
      q.w = MergeOne{t.W[i], t.ldw[i], t.S[i], t.d[i], t.k[i], t.seed[i], t.stream[i]};
      q.local = task - t.t_off[i];
    }
  }
  return q;
}

template <int NKS, bool GAUSS, bool MASKED, int kWaves, int NT, class MT>
__global__ __launch_bounds__(64 * kWaves) void merge_kernel(MT tab, int r, float scale, float cr) {
  constexpr int RP = 32 * NKS;    // r padded to whole K steps
  constexpr int LDA = RP + 8;     // bf16 per LDS column (+16 B against conflicts)
  constexpr int WR = 16 * NT;     // W rows per wave
  // two A slices fit next to the other buffers (up to 112 KB in all)
  constexpr bool kDouble = NKS <= 4 || NT <= 2;
  __shared__ __attribute__((aligned(16))) uint16_t At[(kDouble ? 2 : 1) * kPassCols * LDA];
  __shared__ __attribute__((aligned(16))) uint64_t sgn[GAUSS ? 1 : 4 * RP];
  // Per-wave staging of one pass's results (WR rows x 64 columns) for
  // row-contiguous stores (interior tiles only): fp32 products (row stride
  // kStRowF floats) where W moves in whole lines (NT = 1), else bf16 results
  // (row stride kStRow).
  constexpr bool kLines = NT == 1 && !GAUSS;
  constexpr int kStRow = kPassCols + 8;
  constexpr int kStRowF = kPassCols + 4;
  constexpr int kStageBytes = kLines ? WR * kStRowF * 4 : WR * kStRow * 2;
  __shared__ __attribute__((aligned(16))) unsigned char stage_raw[kWaves * kStageBytes];
  uint16_t* const stage = reinterpret_cast<uint16_t*>(stage_raw);
  float* const stagef = reinterpret_cast<float*>(stage_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 15;   // A-operand row (column slot) and B/D column (row)
  const SignMasks smk = sign_masks();
  const int g = lane >> 4;   // K group for operands, row group for D
  // Flat grid over every weight's tiles, column block fastest, so
  // neighbouring work-groups share rows.  Whole-line tiles: each XCD takes one
  // contiguous run of tasks (whole row blocks, so its L2 fetches those S rows
  // once).  Others: column blocks rotated over the XCDs.
  const int task = kLines ? xcd_runs((int)blockIdx.x, (int)gridDim.x) : (int)blockIdx.x;
  const MergeSel sel = select_weight(tab, task);
  uint16_t* __restrict__ W = sel.w.W;
  const int64_t ldw = sel.w.ldw;
  const float* __restrict__ S = sel.w.S;
  const int d = sel.w.d;
  const int k = sel.w.k;
  const uint64_t seed = sel.w.seed;
  const uint64_t stream = sel.w.stream;
  const int local = sel.local;
  const int n_cb = (k + kMergeCols - 1) / kMergeCols;
  const int rblk = local / n_cb;
  const int cb = kLines ? local % n_cb : xcd_spread(local % n_cb, rblk, n_cb);
  const int col0 = cb * kMergeCols;
  const int row0 = rblk * (WR * kWaves) + wave * WR;
  const int n_pass = min(kMergeCols / kPassCols, (k - col0 + kPassCols - 1) / kPassCols);
  // Work-groups holding the ragged last row block or a ragged last column
  // pass run the masked body; all others the plain one (both are
  // instantiated in a MASKED kernel, so one ragged edge no longer slows
  // every work-group).
  auto body = [&](auto masked_c) {
    constexpr bool M = decltype(masked_c)::value;
    constexpr bool kPreW = kLines && !M;

    // S operands: rows row0 + 16 nt + m, K = r columns 32 ks + 8 g + (0..7),
    // as hi/lo bf16.  They do not depend on the column pass and stay in
    // registers (4 NT NKS u32x4 per lane: large ranks use NT = 2 to fit); with
    // NT = 4 and r > 64 they are rebuilt per pass (L2 hits).
    constexpr bool kHoistS = NKS <= 2 || NT <= 2;
    // rows of this wave all inside d, r a multiple of 32 and S 16-byte
    // aligned (the ABI asks only for 4): plain float4 loads.  A rank that is
    // not a multiple of 32 (or an S that is not 16-byte aligned) needs only
    // the scalar loads below to clear its K tail; they run once, before the
    // passes, so such calls still take the unmasked kernel.
    const bool s_vec = (r % 32) == 0 && (reinterpret_cast<uintptr_t>(S) & 15) == 0;
    const bool s_fast = !M && s_vec;
    auto s_raw = [&](int nt, int ks, float v[8]) {
      const int row = row0 + 16 * nt + m;
      if (s_fast) {
        const f32x4* sp = reinterpret_cast<const f32x4*>(S + (int64_t)row * r + 32 * ks + 8 * g);
        const f32x4 a = sp[0], b = sp[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = a[e];
          v[4 + e] = b[e];
        }
      } else if (s_vec) {   // only rows past d to clear
        f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
        if (row < d) {
          const f32x4* sp = reinterpret_cast<const f32x4*>(S + (int64_t)row * r + 32 * ks + 8 * g);
          a = sp[0];
          b = sp[1];
        }
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
    };
    auto s_split = [&](const float v[8], u32x4& hi, u32x4& lo) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint16_t h0, l0, h1, l1;
        split_bf16(v[2 * p], h0, l0);
        split_bf16(v[2 * p + 1], h1, l1);
        hi[p] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[p] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
    };
    auto s_operands = [&](int nt, int ks, u32x4& hi, u32x4& lo) {
      float v[8];
      s_raw(nt, ks, v);
      s_split(v, hi, lo);
    };
    u32x4 sh[NT][kHoistS ? NKS : 1], sl[NT][kHoistS ? NKS : 1];

    // Sign basis: thread tid < RP / 2 draws the Philox blocks of A rows 2 tid
    // and 2 tid + 1 for this 256-column block and parks their words in LDS,
    // word-major (sgn[q * RP + i] = word q of row i: columns 64 q .. 64 q + 63).
    auto sign_words = [&]() {
      if (!GAUSS && tid < RP / 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = 2 * tid + h;
          Words4 b = {{0, 0, 0, 0}};
          if (i < r) b = sign_block(seed, stream, (uint64_t)cb, (uint64_t)i);
#pragma unroll
          for (int q = 0; q < 4; ++q) sgn[q * RP + i] = b.w[q];
        }
      }
    };

    // A slice of pass p into LDS: buf[col * LDA + i] = A[i][col0 + 64 p + col].
    // Sign basis: every thread takes (8-row group G, column c) jobs: it reads the
    // eight words of rows 8G .. 8G + 7 (one broadcast read per wave), gathers
    // their bit c into one byte and expands it to eight +-1 bf16 (rows >= r: 0).
    auto build_A = [&](int pass, uint16_t* buf) {
      const int c0 = col0 + pass * kPassCols;
      if (GAUSS) {
        for (int job = tid; job < RP * (kPassCols / 4); job += 64 * kWaves) {
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
      } else {
        constexpr int kJobs = kPassCols * (RP / 8);
#pragma unroll
        for (int job = tid; job < kJobs; job += 64 * kWaves) {
          const int c = job & (kPassCols - 1);
          const int grp = job / kPassCols;
          const uint32_t* wp = reinterpret_cast<const uint32_t*>(&sgn[pass * RP + 8 * grp]);
          const int half = c >> 5;           // which dword of each 64-bit word
          const int bit = c & 31;
          uint32_t byte = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) byte |= ((wp[2 * e + half] >> bit) & 1u) << e;
          u32x4 v = signs_to_bf16x8(byte, smk);
          const int valid = r - 8 * grp;     // rows of this group below r
          if (valid < 8) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t keep = (2 * q < valid ? 0x0000FFFFu : 0u) |
                                    (2 * q + 1 < valid ? 0xFFFF0000u : 0u);
              v[q] &= keep;
            }
          }
          *reinterpret_cast<u32x4*>(&buf[c * LDA + 8 * grp]) = v;
        }
      }
    };

    // This lane's W elements of pass p: rows row0 + 16 nt + m, columns
    // col0 + 64 p + 16 g + (0..15).  Rows past d are read from row d - 1 and
    // never stored; columns past k read as zero.
    auto load_W = [&](int pass, u32x4 wv[NT][2]) {
      const int c0 = col0 + pass * kPassCols;
      const int wc = c0 + 16 * g;
      if (!M && kLines) {
        // whole lines: rows row0 + 8 h + lane / 8, columns c0 + 8 (lane % 8) .. + 7
#pragma unroll
        for (int h = 0; h < 2; ++h)
          wv[0][h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
              W + (int64_t)(row0 + 8 * h + (lane >> 3)) * ldw + c0 + 8 * (lane & 7)));
      } else if (!M) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint16_t* wr = W + (int64_t)(row0 + 16 * nt + m) * ldw;
          wv[nt][0] = load_bf16x8(wr, wc);
          wv[nt][1] = load_bf16x8(wr, wc + 8);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
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
    auto do_pass = [&](int pass, u32x4 (&wcur)[NT][2], u32x4 (&wnxt)[NT][2]) {
      if (!kDouble && pass > 0) {
        __syncthreads();          // every wave is done reading the previous slice
        build_A(pass, buf0);
      }
      __syncthreads();            // slice `pass` is complete
      if (pass + 1 < n_pass) {
        if (!kPreW) {
          load_W(pass + 1, wnxt);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (kDouble) build_A(pass + 1, (pass & 1) ? buf0 : buf1);
      }
      const uint16_t* cur_buf = (kDouble && (pass & 1)) ? buf1 : buf0;

      // MFMA: acc[t][nt] rows m' = 4 g' + v map to columns c0 + 16 g' + 4 t + v.
      f32x4 acc[4][NT];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 bh[NT], bl[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
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
          for (int nt = 0; nt < NT; ++nt) {
            acc[t][nt] = mfma16(a, bh[nt], acc[t][nt]);
            acc[t][nt] = mfma16(a, bl[nt], acc[t][nt]);
          }
        }
      }

      // Update and store.
      const int wc = col0 + pass * kPassCols + 16 * g;
      if constexpr (!M && kLines) {
        // products to the wave's fp32 stage (row m, columns 16 g + 4 t + v),
        // back in whole-line order (row 8 h + lane / 8, columns 8 (lane % 8)
        // .. + 7), subtracted from W there, rounded once and stored.  A wave
        // only touches its own stage and its LDS operations complete in
        // order, so no barrier is needed.
        float* st = stagef + wave * (WR * kStRowF);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          *reinterpret_cast<f32x4*>(st + m * kStRowF + 16 * g + 4 * t) = acc[t][0];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rr = 8 * h + (lane >> 3);
          const float* src = st + rr * kStRowF + 8 * (lane & 7);
          const f32x4 p0 = *reinterpret_cast<const f32x4*>(src);
          const f32x4 p1 = *reinterpret_cast<const f32x4*>(src + 4);
          const float pr[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            o[q] = pack_bf16x2(bf16_lo(wcur[0][h][q]) - scale * pr[2 * q],
                               bf16_hi(wcur[0][h][q]) - scale * pr[2 * q + 1]);
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(
              W + (int64_t)(row0 + rr) * ldw + col0 + pass * kPassCols + 8 * (lane & 7)));
        }
        return;
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
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
        if constexpr (!M) {
          uint16_t* stg = stage + (wave * WR + 16 * nt + m) * kStRow + 16 * g;
          *reinterpret_cast<u32x4*>(stg) = out[0];
          *reinterpret_cast<u32x4*>(stg + 8) = out[1];
        } else if (row < d) {
          uint16_t* wr = W + (int64_t)row * ldw;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int cbeg = wc + 8 * hh;
            if (!M || cbeg + 8 <= k) {
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
      // Interior tiles: the wave reads its WR x 64 results back row by row,
      // eight lanes per row, so every store writes whole 128-byte lines (stores
      // of half lines, as the MFMA layout gives them, measured ~10 % slower).
      // A wave only touches its own staging rows and LDS operations of a wave
      // complete in order, so no barrier is needed.
      if constexpr (!M) {
        const int pc = lane & 7;
#pragma unroll
        for (int i = 0; i < WR / 8; ++i) {
          const int rr = 8 * i + (lane >> 3);
          const u32x4 v =
              *reinterpret_cast<const u32x4*>(stage + (wave * WR + rr) * kStRow + 8 * pc);
          *reinterpret_cast<u32x4*>(W + (int64_t)(row0 + rr) * ldw + col0 + pass * kPassCols +
                                    8 * pc) = v;
        }
      }
    };

    // Prologue: start the loads first (S rows, then the W elements of pass 0),
    // regenerate the signs and the first A slice while they are in flight, and
    // only then wait for S.
    u32x4 wa[NT][2], wb[NT][2];
    float sraw[NT][kHoistS ? NKS : 1][8];
    if constexpr (kHoistS) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) s_raw(nt, ks, sraw[nt][ks]);
    }
    // Whole-line interior tiles load the W of all four passes up front (8
    // registers per pass; the loads of a short last column block re-read its
    // last pass), others one pass ahead.
    u32x4 wall[kPreW ? 4 : 1][NT][2];
    if constexpr (kPreW) {
#pragma unroll
      for (int ps = 0; ps < 4; ++ps) load_W(ps < n_pass ? ps : n_pass - 1, wall[ps]);
    } else {
      load_W(0, wa);
    }
    __builtin_amdgcn_sched_barrier(0);
    sign_words();
    __syncthreads();
    build_A(0, buf0);
    if constexpr (kHoistS) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) s_split(sraw[nt][ks], sh[nt][ks], sl[nt][ks]);
    }
    if constexpr (kPreW) {
      do_pass(0, wall[0], wb);
      if (n_pass > 1) do_pass(1, wall[1], wa);
      if (n_pass > 2) do_pass(2, wall[2], wb);
      if (n_pass > 3) do_pass(3, wall[3], wa);
    } else {
      do_pass(0, wa, wb);
      if (n_pass > 1) do_pass(1, wb, wa);
      if (n_pass > 2) do_pass(2, wa, wb);
      if (n_pass > 3) do_pass(3, wb, wa);
    }
  };
  const bool edge = MASKED && ((rblk + 1) * (WR * kWaves) > d ||
                               col0 + n_pass * kPassCols > k);
  if (edge)
    body(std::true_type{});
  else
    body(std::false_type{});
}

// Rows per work-group and per wave (16 NT).  Up to r = 64 with the sign
// basis: 128 rows, eight waves of 16.  A work-group of the d = k = 4096 layer
// then moves 64 KB of W each way and two of them share a CU, so 16 waves per
// CU keep W loads in flight (measured 16.9 -> 12.9 us against 256 rows in four
// waves of 64, about the rate of a device copy).  The Gaussian basis rebuilds
// its A slices from Philox and Box-Muller per work-group, so it keeps 256 rows
// and runs them as sixteen waves of 16 (27.4 -> 21.6 us).  Larger ranks: 256
// rows, eight waves of 32, so each lane's S operands (4 NT NKS u32x4) stay in
// registers for all four column passes instead of being re-read and re-split
// per pass (16 waves of 16 rows spill and ran 15-20 % slower at r = 256; at
// r = 128 the small-rank shapes measured the same).
constexpr int merge_rows(int nks, bool gauss) { return nks <= 2 && !gauss ? 128 : 256; }
constexpr int merge_nt(int nks) { return nks <= 2 ? 1 : 2; }
constexpr int merge_waves(int nks, bool gauss) {
  return merge_rows(nks, gauss) / (16 * merge_nt(nks));
}

template <int NKS, bool MASKED, class MT>
void launch_merge_m(const MT& tab, int r, bool gauss, float scale, float cr, hipStream_t s,
                    dim3 grid) {
  constexpr int kNT = merge_nt(NKS);
  if (gauss) {
    constexpr int kW = merge_waves(NKS, true);
    hipLaunchKernelGGL((merge_kernel<NKS, true, MASKED, kW, kNT, MT>), grid, dim3(64 * kW), 0, s,
                       tab, r, scale, cr);
  } else {
    constexpr int kW = merge_waves(NKS, false);
    hipLaunchKernelGGL((merge_kernel<NKS, false, MASKED, kW, kNT, MT>), grid, dim3(64 * kW), 0, s,
                       tab, r, scale, cr);
  }
}

template <int NKS>
hipError_t launch_merge_t(const MergeItem* items, int n, int r, bool gauss, float scale,
                          float cr, hipStream_t s) {
  const int rows = merge_rows(NKS, gauss);
  int64_t tasks = 0;
  // unmasked when every row block is whole and every 64-column pass is whole
  // (a short last column block just runs fewer passes); one ragged weight
  // makes the launch masked, and only its edge work-groups take the masked
  // body
  bool masked = false;
  for (int i = 0; i < n; ++i) {
    tasks += ((items[i].k + kMergeCols - 1) / kMergeCols) * ((items[i].d + rows - 1) / rows);
    masked = masked || (items[i].d % rows) != 0 || (items[i].k % kPassCols) != 0;
  }
  if (tasks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tasks);
  if (n == 1) {
    const MergeItem& m = items[0];
    const MergeOne one{m.W, m.ldw, m.S, (int)m.d, (int)m.k, m.seed, m.stream};
    if (masked) launch_merge_m<NKS, true>(one, r, gauss, scale, cr, s, grid);
    else launch_merge_m<NKS, false>(one, r, gauss, scale, cr, s, grid);
    return hipGetLastError();
  }
  MergeTable tab{};
  tab.n = n;
  int64_t t = 0;
  for (int i = 0; i < n; ++i) {
    const MergeItem& m = items[i];
    tab.t_off[i] = (int)t;
    t += ((m.k + kMergeCols - 1) / kMergeCols) * ((m.d + rows - 1) / rows);
    tab.W[i] = m.W;
    tab.ldw[i] = m.ldw;
    tab.S[i] = m.S;
    tab.d[i] = (int)m.d;
    tab.k[i] = (int)m.k;
    tab.seed[i] = m.seed;
    tab.stream[i] = m.stream;
  }
  tab.t_off[n] = (int)t;
  if (masked) launch_merge_m<NKS, true>(tab, r, gauss, scale, cr, s, grid);
  else launch_merge_m<NKS, false>(tab, r, gauss, scale, cr, s, grid);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeItem* items, int n, int r, int kind, float alpha, float eta,
                        hipStream_t s) {
  if (n < 1 || n > kMaxMerge) return hipErrorInvalidValue;
  const bool gauss = kind == 1;
  const float cr = sign_scale(r);
  const float step = alpha * eta;             // fp32 product, as documented
  const float scale = gauss ? step : step * cr;
  const int nks = (r + 31) / 32;
  switch (nks <= 1 ? 1 : nks <= 2 ? 2 : nks <= 4 ? 4 : 8) {
    case 1: return launch_merge_t<1>(items, n, r, gauss, scale, cr, s);
    case 2: return launch_merge_t<2>(items, n, r, gauss, scale, cr, s);
    case 4: return launch_merge_t<4>(items, n, r, gauss, scale, cr, s);
    default: return launch_merge_t<8>(items, n, r, gauss, scale, cr, s);
  }
}

}  // namespace logra
