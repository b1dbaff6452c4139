// logra_sketch_accumulate: S += dY^T (X A^T) for one microbatch, on gfx950.
//
// [LoGRA] (wispaper.ai summary of "LoGRA: Scaling LLM Reinforcement Learning
// with Low-Rank Gradient Sketches"), section Sketch: each microbatch's
// contribution to the d x r sketch S = G A^T is accumulated in fp32 by
// projecting the layer inputs first and only then multiplying with the
// backward derivatives, so the d x k gradient is never formed.
//
// Kernels on the caller's stream (no cross-work-group synchronisation inside
// any of them: on this part an agent-scope fence per work-group costs far more
// than an extra launch):
//   project    P = c * X A^T (T x r).  One work-group per 32 tokens
//              (project_kernel), or per 64 tokens from r = 64 when that still
//              fills the chip or the basis is Gaussian (project_tile_kernel);
//              its waves split k in 256-column chunks, which reach LDS through
//              direct global->LDS loads (whole cache lines per instruction)
//              while the previous chunk is multiplied.  For the sign basis
//              each lane regenerates the sign bits of its A row in registers
//              from Philox (one block per row and chunk) and expands them to
//              bf16 +-1 MFMA operands, so A never touches memory.  Products
//              with +-1 are exact; 32x32x16 bf16 MFMA accumulates in fp32;
//              the waves' partial sums meet in LDS in a fixed order.  P is
//              stored as a hi/lo bf16 pair in the accumulate kernel's operand
//              order (one contiguous 1 KB block per 32 tokens x 16 r columns).
//   accumulate S += dY^T P.  A work-group owns 16*Q columns of d and a range
//              of 32-token steps (accumulate_kernel).  Each lane loads an
//              8-token x Q-column block of dY with row-contiguous loads and
//              transposes it in registers (v_perm_b32), giving K = token
//              operands for 16x16x32 MFMA against P_hi and P_lo.  Waves split
//              the steps (and, above r = 64, the rank) and are summed in LDS
//              in a fixed order.  From r = 128 at T >= 16384 a work-group
//              instead owns 2 or 4 such column groups and all of r, with dY
//              and P staged once per step in LDS for all its waves
//              (accumulate_wide_kernel).  Tasks (split, column group) are
//              numbered split-major and dealt to the XCDs in contiguous runs,
//              so each XCD's L2 fetches the P tiles of one or two splits.
//              With several work-groups along T each writes its partial
//              tile, and
//   finalize   adds the partial tiles to S in split order.  S is therefore
//              bit-reproducible.  With the overwrite flag the kernel that
//              writes S stores the result instead of adding it.
// Deferred calls (defer) leave S alone: their contribution stays in the
// partial tiles, which a later call (pending) adds its own to, split by
// split; only a call without defer runs the finalize.  A step of several
// microbatches then pays for one split reduction instead of one per call.
// The Gaussian basis is first written once per call as a bf16 r x k matrix in
// the workspace (Box-Muller per entry is too costly to repeat per token
// block) and the project kernel reads its operand tiles from there.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace logra {

namespace {

// Waves per project work-group: eight (two per SIMD, 128 KB of X staging)
// unless the accumulators of a large rank need the larger register budget.
constexpr int proj_waves(int nb) { return nb <= 4 ? 8 : 4; }

// Accumulate work-groups: eight waves (two per SIMD), each holding a tile of
// 128 d columns x up to 64 r columns (NB16 blocks of 16) of the sketch, with
// its steps' P operands in a per-wave two-slot LDS ring (8 waves x 16 KB).
// Ranks above 64 split r across the waves (2 or 4 ways) rather than shrink
// the d tile, so every P byte brought to a CU still meets 128 d columns.
constexpr int kAccWaves = 8;
constexpr int kAccQ = 8;                                      // d columns per lane / 16
constexpr int acc_nbw(int nb16) { return nb16 < 4 ? nb16 : 4; }   // r blocks per wave
constexpr int acc_rsplit(int nb16) { return nb16 / acc_nbw(nb16); }

// ------------------------------------------------------------------ project
// X reaches LDS by direct global->LDS loads (global_load_lds_dwordx4): each
// instruction moves 1 KB, four token rows x 256 contiguous bytes, so every
// cache line is fetched by one instruction (register loads in MFMA operand
// order would touch 32 rows per instruction and refetch each line 8 times).
// A wave stages one 256-column chunk as two 128-column halves of 8 KB, each
// 32 rows x 16 pieces of 16 bytes; piece j of row t sits at slot j ^ (t % 16)
// so the MFMA operand reads (row = lane % 32) hit distinct banks.
constexpr int kHalfCols = 128;
constexpr int kHalfBytes = 32 * kHalfCols * 2;

typedef __attribute__((address_space(3))) void lds_void;

// Element offset of the P operand block (step, 16-column block nb, half hl)
// in the tiled P buffer.  Inside a block, lane slot l = 16 g4 + n holds the
// eight tokens 32 step + 8 g4 + (0..7) of r column 16 nb + n.
__device__ __forceinline__ int64_t p_block(int step, int nb, int hl, int nb16) {
  return ((int64_t)(step * nb16 + nb) * 2 + hl) * 512;
}

// The input groups of a projection launch as its first kernel argument.
// ProjOne: the one group of a single or shared call (the launch arguments
// stay as small as separate parameters; a launch's cost was measured to grow
// with its argument bytes).  ProjTable: the groups of a layer call; group g
// owns work-groups g n_blk .. (g + 1) n_blk - 1, each group with its own X,
// k, A (seed, stream; or the Gaussian basis Ab with row stride lda) and P.
struct ProjOne {
  const uint16_t* X;
  int64_t ldx;
  int k;
  uint64_t seed;
  uint64_t stream;
  const uint16_t* Ab;
  int64_t lda;
  uint16_t* Pt;
};
struct ProjTable {
  int n;
  int n_blk;
  const uint16_t* X[kMaxGroups];
  int64_t ldx[kMaxGroups];
  int k[kMaxGroups];
  uint64_t seed[kMaxGroups];
  uint64_t stream[kMaxGroups];
  const uint16_t* Ab[kMaxGroups];
  int64_t lda[kMaxGroups];
  uint16_t* Pt[kMaxGroups];
};

// The group of work-group bx, its block index within the group (bl) and the
// group's block count.  Table entries are chosen with compares and selects
// on constant indices (a variable index into the by-value argument would copy
// it to scratch memory).
struct ProjSel {
  const uint16_t* X;
  int64_t ldx;
  int k;
  uint64_t seed;
  uint64_t stream;
  const uint16_t* Ab;
  int64_t lda;
  uint16_t* Pt;
  int bl;
  int n_blk;
};
__device__ __forceinline__ ProjSel select_group(const ProjOne& t, int bx) {
  return ProjSel{t.X, t.ldx, t.k, t.seed, t.stream, t.Ab, t.lda, t.Pt, bx, (int)gridDim.x};
}
// (Each later group that the block index reaches overrides the fields: the
// compares stay compares.  Written as "entry i == chosen index" the compiler
// turns the selects back into a variable index and copies the table to
// scratch memory.)
__device__ __forceinline__ ProjSel select_group(const ProjTable& t, int bx) {
  ProjSel q{t.X[0], t.ldx[0], t.k[0], t.seed[0], t.stream[0], t.Ab[0], t.lda[0], t.Pt[0], bx,
            t.n_blk};
#pragma unroll
  for (int i = 1; i < kMaxGroups; ++i) {
    if (i < t.n && bx >= i * t.n_blk) {
      q.X = t.X[i];
      q.ldx = t.ldx[i];
      q.k = t.k[i];
      q.seed = t.seed[i];
      q.stream = t.stream[i];
      q.Ab = t.Ab[i];
      q.lda = t.lda[i];
      q.Pt = t.Pt[i];
      q.bl = bx - i * t.n_blk;
    }
  }
  return q;
}
#define LOGRA_GROUP_FIELDS(gs)                       \
  const uint16_t* __restrict__ X = (gs).X;           \
  const int64_t ldx = (gs).ldx;                      \
  const int k = (gs).k;                              \
  const uint64_t seed = (gs).seed;                   \
  const uint64_t stream = (gs).stream;               \
  const uint16_t* __restrict__ Ab = (gs).Ab;         \
  const int64_t lda = (gs).lda;                      \
  uint16_t* __restrict__ Pt = (gs).Pt

template <int NB, bool GAUSS, bool MASKED, int kProjWaves, class PT>
__global__ __launch_bounds__(64 * kProjWaves) void project_kernel(PT tab, int T, int rp, float c) {
  __shared__ __attribute__((aligned(16))) unsigned char stage0[kProjWaves][kHalfBytes];
  __shared__ __attribute__((aligned(16))) unsigned char stage1[kProjWaves][kHalfBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m = lane & 31;  // A-operand row (token) and B-operand column (A row)
  const int h = lane >> 5;  // which 64-column quarter of a half this lane feeds
  const ProjSel gs = select_group(tab, (int)blockIdx.x);
  LOGRA_GROUP_FIELDS(gs);
  const int step = xcd_spread(gs.bl, gs.bl >> 3, gs.n_blk);
  const int t0 = step * 32;
  const SignMasks smk = sign_masks();
  const int n_chunks = (k + 255) >> 8;
  unsigned char* buf0 = stage0[wave];
  unsigned char* buf1 = stage1[wave];

  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[nb][v] = 0.0f;
  }

  // Half hc of chunk cnk -> dst.  Instruction i: lane l brings piece
  // (l % 16) ^ (row % 16) of row 4 i + l / 16.  Rows >= T re-read row T - 1
  // and pieces past k re-read the row's first piece; both are cleared when
  // read back.
  auto issue = [&](int cnk, int hc, unsigned char* dst) {
    const int colbase = cnk * 256 + hc * kHalfCols;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + (lane >> 4);
      const int j = (lane & 15) ^ (row & 15);
      int t = t0 + row;
      int col = colbase + 8 * j;
      if (t0 + 32 > T) t = t < T ? t : T - 1;                       // ragged block only
      if (MASKED && (cnk + 1) * 256 > k) col = col < k ? col : 0;   // ragged chunk only
      lds_dma16_nt((const void*)(X + (int64_t)t * ldx + col), lds_addr(dst + i * 1024));
    }
  };

  // Sign words of A row 32 nb + m for chunk ch: word 2 hc + h feeds half hc.
  // With two or more 32-row blocks the lane halves draw different blocks
  // (half h draws block 2 j + h) and swap the words the other half needs, so
  // no Philox block is computed twice.
  uint64_t sw[NB][2];
  auto sign_words = [&](int ch) {
    if constexpr (NB == 1) {
      const Words4 blk = sign_block(seed, stream, (uint64_t)ch, (uint64_t)m);
      sw[0][0] = h ? blk.w[1] : blk.w[0];
      sw[0][1] = h ? blk.w[3] : blk.w[2];
    } else {
#pragma unroll
      for (int j = 0; j < NB / 2; ++j) {
        const Words4 blk =
            sign_block(seed, stream, (uint64_t)ch, (uint64_t)((2 * j + h) * 32 + m));
        const uint64_t r0 = swap_halves64(h ? blk.w[0] : blk.w[1]);
        const uint64_t r2 = swap_halves64(h ? blk.w[2] : blk.w[3]);
        sw[2 * j][0] = h ? r0 : blk.w[0];
        sw[2 * j][1] = h ? r2 : blk.w[2];
        sw[2 * j + 1][0] = h ? blk.w[1] : r0;
        sw[2 * j + 1][1] = h ? blk.w[3] : r2;
      }
    }
  };

  // K assignment: in step s of half hc, lane half h carries columns
  // 256 ch + 128 hc + 64 h + 8 s + (0..7) - byte s of sign word 2 hc + h.
  // Columns past k (ragged k only, MASKED) are cleared in the last chunk.
  // Token rows past T need no mask: their copies re-read row T - 1 and the
  // store below writes zeros for them.
  auto compute = [&](int ch, int hc, const unsigned char* buf) {
    const int colq = ch * 256 + hc * kHalfCols + 64 * h;
    const bool edge = MASKED && (ch + 1) * 256 > k;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int slot = (8 * h + s) ^ (m & 15);
      u32x4 a = *reinterpret_cast<const u32x4*>(buf + m * (kHalfCols * 2) + slot * 16);
      if (edge) a &= keep_mask8(k - (colq + 8 * s));
      if constexpr (GAUSS) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const u32x4 b = *reinterpret_cast<const u32x4*>(
              Ab + (int64_t)(nb * 32 + m) * lda + colq + 8 * s);
          acc[nb] = mfma32(a, b, acc[nb]);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint32_t byte = (uint32_t)(sw[nb][hc] >> (8 * s)) & 0xFFu;
          acc[nb] = mfma32(a, signs_to_bf16x8(byte, smk), acc[nb]);
        }
      }
    }
  };

  // Per wave: logical chunks wave, wave + W, ...; the two halves of the next
  // chunk load while the current one is multiplied.  The copies are issued
  // from inline assembly (lds_dma16), so the compiler's wait-count pass does
  // not make the reads of one half wait for the copy just issued into the
  // other; the kernel waits for each half itself: 8 copies per half, in
  // issue order.  Each work-group starts
  // its walk along k at a different chunk (physical chunk = logical + step,
  // mod n_chunks): work-groups that run in lock step would otherwise all read
  // the same byte range of their rows at the same time, and HBM channels are
  // interleaved by address within a row, so half of them would sit idle.
  const int rot = step % n_chunks;
  auto phys = [&](int c) { c += rot; return c < n_chunks ? c : c - n_chunks; };
  int ch = wave;
  if (ch < n_chunks) {
    issue(phys(ch), 0, buf0);
    issue(phys(ch), 1, buf1);
  }
  for (; ch < n_chunks; ch += kProjWaves) {
    const int pc = phys(ch);
    if constexpr (!GAUSS) sign_words(pc);
    const bool more = ch + kProjWaves < n_chunks;
    vm_wait<8>();          // half 0 landed; half 1's copies may be in flight
    compute(pc, 0, buf0);
    if (more) {
      lgkm_wait0();        // this wave's reads of buf0 are done
      issue(phys(ch + kProjWaves), 0, buf0);
      vm_wait<8>();        // half 1 landed; the next half 0 stays in flight
    } else {
      vm_wait<0>();
    }
    compute(pc, 1, buf1);
    if (more) {
      lgkm_wait0();
      issue(phys(ch + kProjWaves), 1, buf1);
    }
  }

  // Sum the waves' partial P in a fixed order (w0 + w1 + ...) and store the
  // hi/lo pair in the tiled layout.  Thread (n_out, tg) owns the TPT tokens
  // TPT tg .. TPT tg + TPT - 1 of A row 32 nb + n_out.  The staging buffers
  // are free (every load was consumed above) and hold the partial sums.
  constexpr int TPT = 16 / kProjWaves;     // tokens per thread: 2 or 4
  static_assert(kProjWaves * 32 * 33 * 4 <= kProjWaves * kHalfBytes, "red fits");
  float (*red)[32 * 33] = reinterpret_cast<float (*)[32 * 33]>(&stage0[0][0]);
  const int n_out = tid & 31;
  const int tg = tid >> 5;
  const int nb16 = rp >> 4;
  __syncthreads();
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 8 * (v >> 2) + 4 * h + (v & 3);
      red[wave][row * 33 + m] = acc[nb][v];
    }
    __syncthreads();
    const int i = nb * 32 + n_out;
    if (i < rp) {
      uint16_t hi[TPT], lo[TPT];
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int idx = (TPT * tg + u) * 33 + n_out;
        float p = red[0][idx];
#pragma unroll
        for (int w = 1; w < kProjWaves; ++w) p += red[w][idx];
        if (t0 + TPT * tg + u >= T) p = 0.0f;      // token past T
        split_bf16(p * c, hi[u], lo[u]);
      }
      const int u0 = TPT * tg;                 // first token within the step
      const int64_t slot = (int64_t)(((u0 >> 3) * 16 + (i & 15)) * 8 + (u0 & 7));
      uint16_t* ph = Pt + p_block(step, i >> 4, 0, nb16) + slot;
      uint16_t* pl = Pt + p_block(step, i >> 4, 1, nb16) + slot;
#pragma unroll
      for (int u = 0; u < TPT; u += 2) {
        *reinterpret_cast<uint32_t*>(ph + u) = (uint32_t)hi[u] | ((uint32_t)hi[u + 1] << 16);
        *reinterpret_cast<uint32_t*>(pl + u) = (uint32_t)lo[u] | ((uint32_t)lo[u + 1] << 16);
      }
    }
    __syncthreads();
  }
}

// Projection with 32 TB tokens per work-group, for r >= 64 (chosen by
// tile_blocks below).  TB = 2: waves 0-3 and 4-7 take the two halves of r
// (NBW 32-row blocks of A each) over the same 256-column chunks of k (chunk
// lane = wave mod 4), and each chunk lane's 64 X rows reach LDS once for both
// halves, 32 rows from each of its two waves.  A wave multiplies every sign
// (or Gaussian) operand it builds with both 32-token blocks, so the Philox
// words and the +-1 expansion cost half as much per product as in
// project_kernel, whose waves cover one 32-token block (at r = 256 that
// kernel issues ~24 VALU instructions per MFMA).  TB = 4 (from r = 128, where
// its work-groups still fill the chip): 128 tokens, two chunk lanes x four r
// parts, so every operand a wave builds meets four token blocks.  Either way
// 128 KiB of staging.  The half-chunk steps of all lanes run in lock step
// with one barrier each: after it, a wave's own copy and its partners' have
// landed and every wave is done reading the other buffer, which is refilled
// while this step is multiplied.
constexpr int tile_lanes(int tb) { return tb == 2 ? 4 : 2; }   // chunk lanes

template <int NBW, bool GAUSS, bool MASKED, int TB, class PT>
__global__ __launch_bounds__(512) void project_tile_kernel(PT tab, int T, int rp, int steps_total,
                                                           float c) {
  static_assert(NBW % 2 == 0 || NBW == 1, "sign words pair 32-row blocks");
  static_assert(TB == 2 || TB == 4, "64- or 128-token tiles");
  constexpr int kLanes = tile_lanes(TB);   // chunk lanes
  constexpr int kRParts = 8 / kLanes;      // r parts (= TB: each wave brings 32 rows)
  constexpr int kTok = 32 * TB;            // tokens per work-group
  static_assert(kRParts == TB, "a chunk lane's waves bring its TB x 32 X rows");
  // [chunk lane][half][kTok rows x 128 columns bf16], 16-byte pieces swizzled by row
  __shared__ __attribute__((aligned(16))) unsigned char stage[kLanes][2][TB * kHalfBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rpart = wave / kLanes;       // which part of r
  const int cl = wave % kLanes;          // chunk lane
  const int m = lane & 31;  // A-operand row (token) and B-operand column (A row)
  const int h = lane >> 5;  // which 64-column quarter of a half this lane feeds
  const ProjSel gs = select_group(tab, (int)blockIdx.x);
  LOGRA_GROUP_FIELDS(gs);
  const int blk = xcd_spread(gs.bl, gs.bl >> 3, gs.n_blk);
  const int t0 = blk * kTok;
  const SignMasks smk = sign_masks();
  const int n_chunks = (k + 255) >> 8;
  const int row_base = rpart * NBW * 32;   // first A row of this wave

  f32x16 acc[TB][NBW];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[tb][nb][v] = 0.0f;

  // This wave's 32 rows (32 rpart ..) of half hc of chunk cnk -> dst, eight
  // direct global->LDS copies of 4 rows x 256 bytes.  Rows >= T re-read row
  // T - 1 and pieces past k re-read the row's first piece; both are cleared
  // when read back.
  auto issue = [&](int cnk, int hc, unsigned char* dst) {
    const int colbase = cnk * 256 + hc * kHalfCols;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 32 * rpart + 4 * i + (lane >> 4);
      const int j = (lane & 15) ^ (row & 15);
      int t = t0 + row;
      int col = colbase + 8 * j;
      if (t0 + kTok > T) t = t < T ? t : T - 1;                     // ragged tile only
      if (MASKED && (cnk + 1) * 256 > k) col = col < k ? col : 0;  // ragged chunk only
      lds_dma16_nt((const void*)(X + (int64_t)t * ldx + col),
                   lds_addr(dst + (32 * rpart + 4 * i) * (kHalfCols * 2)));
    }
  };

  // Sign words of A rows row_base + 32 nb + m for chunk ch (word 2 hc + h
  // feeds half hc); the lane halves draw different row blocks and swap the
  // words the other half needs, as in project_kernel.
  uint64_t sw[NBW][2];
  auto sign_words = [&](int ch) {
    if constexpr (NBW == 1) {
      const Words4 b = sign_block(seed, stream, (uint64_t)ch, (uint64_t)(row_base + m));
      sw[0][0] = h ? b.w[1] : b.w[0];
      sw[0][1] = h ? b.w[3] : b.w[2];
    } else {
#pragma unroll
      for (int j = 0; j < NBW / 2; ++j) {
        const Words4 b =
            sign_block(seed, stream, (uint64_t)ch, (uint64_t)(row_base + (2 * j + h) * 32 + m));
        const uint64_t r0 = swap_halves64(h ? b.w[0] : b.w[1]);
        const uint64_t r2 = swap_halves64(h ? b.w[2] : b.w[3]);
        sw[2 * j][0] = h ? r0 : b.w[0];
        sw[2 * j][1] = h ? r2 : b.w[2];
        sw[2 * j + 1][0] = h ? b.w[1] : r0;
        sw[2 * j + 1][1] = h ? b.w[3] : r2;
      }
    }
  };

  // Columns past k cleared in the ragged last chunk only (MASKED); token
  // rows past T re-read row T - 1 and are zeroed at the store, as in
  // project_kernel.
  // Gaussian basis with one 32-row block per wave (r = 64): the half-step's
  // eight operands come from L2, loaded one half-step ahead into one of two
  // register sets (gb_a / gb_b below) so their latency hides behind the
  // previous half-step's MFMAs; wider Gaussian ranks load them in place.
  constexpr bool kPrefetchB = GAUSS && NBW == 1;
  typedef u32x4 GbSet[kPrefetchB ? 8 : 1];
  auto load_gb = [&](int ch, int hc, GbSet& dst) {
    if constexpr (kPrefetchB) {
      const uint16_t* src = Ab + (int64_t)(row_base + m) * lda + ch * 256 + hc * kHalfCols + 64 * h;
#pragma unroll
      for (int s = 0; s < 8; ++s) dst[s] = *reinterpret_cast<const u32x4*>(src + 8 * s);
    }
  };
  auto compute = [&](int ch, int hc, const unsigned char* buf, const GbSet& gbc) {
    const int colq = ch * 256 + hc * kHalfCols + 64 * h;
    const bool edge = MASKED && (ch + 1) * 256 > k;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int slot = (8 * h + s) ^ (m & 15);
      u32x4 a[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        a[tb] = *reinterpret_cast<const u32x4*>(buf + (32 * tb + m) * (kHalfCols * 2) + slot * 16);
      if (edge) {
        const u32x4 keep = keep_mask8(k - (colq + 8 * s));
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) a[tb] &= keep;
      }
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        u32x4 b;
        if constexpr (kPrefetchB) {
          b = gbc[s];
        } else if constexpr (GAUSS) {
          b = *reinterpret_cast<const u32x4*>(Ab + (int64_t)(row_base + nb * 32 + m) * lda +
                                              colq + 8 * s);
        } else {
          b = signs_to_bf16x8((uint32_t)(sw[nb][hc] >> (8 * s)) & 0xFFu, smk);
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[tb][nb] = mfma32(a[tb], b, acc[tb][nb]);
      }
    }
  };

  // Lane cl takes chunks cl, cl + kLanes, ... (physical chunk = logical +
  // block, mod n_chunks, as in project_kernel); every lane runs
  // 2 ceil(n / kLanes) steps so the barriers match, idling past its last chunk.
  const int rot = blk % n_chunks;
  auto phys = [&](int cc) { cc += rot; return cc < n_chunks ? cc : cc - n_chunks; };
  const int n_mine = cl < n_chunks ? (n_chunks - cl + kLanes - 1) / kLanes : 0;
  const int n_steps = 2 * ((n_chunks + kLanes - 1) / kLanes);
  // One half-step; with the prefetch the loop below runs them in pairs
  // (n_steps is even) so the two operand sets swap roles at compile time.
  GbSet gb_a, gb_b;
  auto half_step = [&](int step, const GbSet& cur, GbSet& nxt) {
    const int jc = step >> 1;
    const int hc = step & 1;
    vm_wait<0>();       // this wave's copies (and operand loads) for the step have landed
    __syncthreads();    // ... and its partner's; the other buffer is free
    const int nj = (step + 1) >> 1;
    if (nj < n_mine) {
      issue(phys(cl + kLanes * nj), (step + 1) & 1, stage[cl][(step + 1) & 1]);
      load_gb(phys(cl + kLanes * nj), (step + 1) & 1, nxt);
    }
    if (jc < n_mine) {
      const int pc = phys(cl + kLanes * jc);
      if constexpr (!GAUSS) {
        if (hc == 0) sign_words(pc);
      }
      lgkm_wait0();
      compute(pc, hc, stage[cl][hc], cur);
    }
  };
  if (n_mine > 0) {
    issue(phys(cl), 0, stage[cl][0]);
    load_gb(phys(cl), 0, gb_a);
  }
  if constexpr (kPrefetchB) {
    for (int step = 0; step < n_steps; step += 2) {
      half_step(step, gb_a, gb_b);
      half_step(step + 1, gb_b, gb_a);
    }
  } else {
    // (unrolled by two, the other variants ran out of registers: the
    // Gaussian r = 256 tile measured 128 -> 164 us)
    for (int step = 0; step < n_steps; ++step) half_step(step, gb_a, gb_b);
  }
  vm_wait<0>();

  // Sum the chunk lanes of each r part in a fixed order (l0 + l1 + ...), one
  // (token block, r block) at a time through LDS, and store the hi/lo pair in
  // the tiled layout.  Thread t: r part t / (512 / kRParts), r column n_out of
  // the block, tokens kTpt tg .. kTpt tg + kTpt - 1.
  constexpr int kThrPart = 512 / kRParts;
  constexpr int kTpt = 32 / (kThrPart / 32);   // tokens per thread: 4 or 8
  static_assert(8 * 32 * 33 * 4 <= (int)sizeof(stage), "reduction buffer fits");
  float (*red)[32 * 33] = reinterpret_cast<float (*)[32 * 33]>(&stage[0][0][0]);
  const int rh = tid / kThrPart;
  const int n_out = tid & 31;
  const int tg = (tid % kThrPart) >> 5;
  const int nb16 = rp >> 4;
  __syncthreads();
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * h + (v & 3);
        red[wave][row * 33 + m] = acc[tb][nb][v];
      }
      __syncthreads();
      const int step = TB * blk + tb;
      const int i = (rh * NBW + nb) * 32 + n_out;   // A row / P column
      if (step < steps_total && i < rp) {
        uint16_t hi[kTpt], lo[kTpt];
#pragma unroll
        for (int u = 0; u < kTpt; ++u) {
          const int idx = (kTpt * tg + u) * 33 + n_out;
          float p = red[rh * kLanes][idx];
#pragma unroll
          for (int w = 1; w < kLanes; ++w) p += red[rh * kLanes + w][idx];
          if (t0 + 32 * tb + kTpt * tg + u >= T) p = 0.0f;   // token past T
          split_bf16(p * c, hi[u], lo[u]);
        }
        const int u0 = kTpt * tg;
        const int64_t slot = (int64_t)(((u0 >> 3) * 16 + (i & 15)) * 8 + (u0 & 7));
        uint16_t* ph = Pt + p_block(step, i >> 4, 0, nb16) + slot;
        uint16_t* pl = Pt + p_block(step, i >> 4, 1, nb16) + slot;
#pragma unroll
        for (int u = 0; u < kTpt; u += 2) {
          *reinterpret_cast<uint32_t*>(ph + u) = (uint32_t)hi[u] | ((uint32_t)hi[u + 1] << 16);
          *reinterpret_cast<uint32_t*>(pl + u) = (uint32_t)lo[u] | ((uint32_t)lo[u + 1] << 16);
        }
      }
      __syncthreads();
    }
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
// dY rows of one 32-token step for lane (m, g4): tokens tb .. tb + 7 x Q
// columns from `col` (tb = 32 step + 8 g4).
template <int Q>
struct DyStage {
  uint32_t R[8][Q / 2];
};

// dY loads go through a buffer resource over the step's rows: the row offset
// e * ldd rides in the scalar offset and the lane's own offset in one 32-bit
// register (the caller guarantees 64 * ldd < 2^32), and rows at or past T
// fall outside the resource and read as zero.  Columns at or past d read the
// row's first group; the kernel zeroes their A operands.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufferDword3 = 0x00020000;   // raw buffer, 32-bit data (gfx9)
// Cache policy of the dY loads: non-temporal (the nt bit).  dY is read once
// per call; measured with no input re-read from the Infinity Cache (a step
// takes other buffers than the step before): the d = k = 4096 step 166.8 ->
// 162.8 us, the 1.5B-shaped layer calls 5-6 % (r = 16) and 1.5-3 % (r = 64)
// faster, a lone call without a chain ~2 % slower.
constexpr int kNonTemporal = 2;

// The lane's fixed part of the offset: row 8 g4 of the step, column col
// (the row's first group when col is past d).
__device__ __forceinline__ int dy_lane_offset(int64_t ldd, int d, int col, int g4) {
  const int c = col < d ? col : 0;
  return (int)(((uint32_t)(8 * g4) * (uint32_t)ldd + (uint32_t)c) * 2u);
}

// valid = false gives a resource of zero bytes: the loads are still issued
// (so every path through a pipeline has the same loads outstanding for the
// compiler's wait counts) but read nothing and return zeros.
template <int Q>
__device__ __forceinline__ void load_dy_stage(const uint16_t* __restrict__ dY,
                                              int64_t ldd, int T, int vo, int step,
                                              DyStage<Q>& st, bool valid = true) {
  const int64_t row0 = (int64_t)step * 32;
  const int64_t rows = T - row0 < 32 ? T - row0 : 32;
  const uint32_t bytes = valid && rows > 0 ? (uint32_t)rows * (uint32_t)ldd * 2u : 0u;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(dY + row0 * ldd), (short)0, (int)bytes, kBufferDword3);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int so = (int)((uint32_t)e * (uint32_t)ldd * 2u);
    uint32_t v[Q / 2];
    if constexpr (Q == 8) {
      const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, so, kNonTemporal);
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = (uint32_t)x[u];
    } else if constexpr (Q == 4) {
      const i32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, vo, so, kNonTemporal);
      v[0] = (uint32_t)x[0];
      v[1] = (uint32_t)x[1];
    } else {
      v[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, vo, so, kNonTemporal);
    }
#pragma unroll
    for (int u = 0; u < Q / 2; ++u) st.R[e][u] = v[u];
  }
}

// Register i = (q * NB16 + nb) * 4 + v of lane (n = lane % 16, g = lane / 16)
// of the accumulators holds d row dc0 + Q (4 g + v) + q, r column 16 nb + n.
template <int Q, int NB16>
__device__ __forceinline__ int acc_drow(int dc0, int i, int ln) {
  return dc0 + Q * (4 * (ln >> 4) + (i & 3)) + i / (NB16 * 4);
}
template <int NB16>
__device__ __forceinline__ int acc_rcol(int i, int ln) {
  return 16 * ((i >> 2) % NB16) + (ln & 15);
}

// Registers per round of the cross-wave sum: 64 when r is split across the
// waves or when a wave holds four r blocks (the P ring then already takes the
// 128 KiB that 64 registers of eight waves need), else 32.
constexpr int acc_round(int nb16) {
  return (acc_rsplit(nb16) > 1 || acc_nbw(nb16) == 4) ? 64 : 32;
}

// LDS bytes of the accumulate kernel: the P ring and the reduction buffer
// share one array.
template <int NB16>
constexpr int acc_lds_bytes() {
  constexpr int ring = kAccWaves * 2 * (acc_nbw(NB16) * 2 * 1024);
  constexpr int red = kAccWaves * acc_round(NB16) * 64 * 4;
  return ring > red ? ring : red;
}

// The outputs of one call as a kernel argument.  Work-group d groups are
// numbered across all outputs; output o owns groups dg_off[o] .. dg_off[o+1].
// OutTable: the outputs of one input group (single and shared calls; their P
// is a separate argument, so the launch arguments stay as small as before).
// LayerOutTable: the outputs of a layer call, each with its group's P.
struct OutTable {
  static constexpr int kN = kMaxShared;
  int n;
  int overwrite;   // S = result instead of S += result (S is not read)
  int pending;     // the partial tiles hold earlier deferred contributions: add to them
  int dg_off[kN + 1];
  int wg_off[kN + 1];   // first accumulate_wide_kernel work-group of each output
  const uint16_t* dY[kN];
  int64_t ldd[kN];
  int d[kN];
  float* S[kN];
};
struct LayerOutTable {
  static constexpr int kN = kMaxOut;
  int n;
  int overwrite;
  int pending;
  int dg_off[kN + 1];
  int wg_off[kN + 1];
  const uint16_t* dY[kN];
  int64_t ldd[kN];
  int d[kN];
  float* S[kN];
  const uint16_t* Pt[kN];   // the P of the output's input group
};

// P of output i: the call's one P, or the output's own.
__device__ __forceinline__ const uint16_t* out_p(const OutTable&, int, const uint16_t* p) {
  return p;
}
__device__ __forceinline__ const uint16_t* out_p(const LayerOutTable& t, int i, const uint16_t*) {
  return t.Pt[i];
}

// The fields of one output, chosen from a table (below).
struct OutSel {
  const uint16_t* dY;
  int64_t ldd;
  int d;
  float* S;
  const uint16_t* Pt;
  int dg_first;
  int dg_end;
  int wg_first;
};
// The output owning global d group dgg (wave-uniform) or accumulate_wide_kernel
// work-group wg (by_wg): each later output that the index reaches overrides
// the fields (compares, not a variable index: see select_group).
template <bool by_wg, class Tab>
__device__ __forceinline__ OutSel select_out_t(const Tab& t, int idx, const uint16_t* p) {
  OutSel q{t.dY[0], t.ldd[0], t.d[0], t.S[0], out_p(t, 0, p), t.dg_off[0], t.dg_off[1],
           t.wg_off[0]};
#pragma unroll
  for (int i = 1; i < Tab::kN; ++i) {
    if (i < t.n && idx >= (by_wg ? t.wg_off[i] : t.dg_off[i])) {
      q.dY = t.dY[i];
      q.ldd = t.ldd[i];
      q.d = t.d[i];
      q.S = t.S[i];
      q.Pt = out_p(t, i, p);
      q.dg_first = t.dg_off[i];
      q.dg_end = t.dg_off[i + 1];
      q.wg_first = t.wg_off[i];
    }
  }
  return q;
}
template <class Tab>
__device__ __forceinline__ OutSel select_out(const Tab& t, int dgg, const uint16_t* p) {
  return select_out_t<false>(t, dgg, p);
}
template <class Tab>
__device__ __forceinline__ OutSel select_out_wg(const Tab& t, int wg, const uint16_t* p) {
  return select_out_t<true>(t, wg, p);
}

// S += dY^T P over a range of 32-token steps for 16 Q columns of d.
// The P operands of each step reach a per-wave two-slot LDS ring by direct
// global->LDS loads issued from inline assembly, so the compiler's wait-count
// pass (which would wait for every outstanding vector load before any LDS
// read) keeps the dY prefetch in flight; the kernel waits for each P slot
// itself with an exact vmcnt.  With r split RS ways, wave w takes r blocks
// NBW (w / L) .. and steps s_begin + (w % L) + L j (L = 8 / RS waves along
// the steps); waves of one r part load the same dY rows (cache hits after
// the first).
template <int Q, int NB16, bool MASKED, class Tab>
__global__ __launch_bounds__(64 * kAccWaves) void accumulate_kernel(
    Tab tab, int T, int r, const uint16_t* __restrict__ Pt1, int steps_total, int steps_per_split,
    float* __restrict__ part) {
  constexpr int DC = 16 * Q;            // d columns per work-group
  constexpr int NREG = Q * NB16 * 4;    // accumulator floats of the tile per lane
  constexpr int NBW = acc_nbw(NB16);    // 16-column r blocks per wave
  constexpr int RS = NB16 / NBW;        // ways r is split across the waves
  constexpr int NREGW = Q * NBW * 4;    // accumulator floats per lane of one wave
  constexpr int kLanes = kAccWaves / RS;     // waves along the steps
  constexpr int CH = acc_round(NB16);        // registers per reduction round
  constexpr int kSlot = NBW * 2 * 1024;      // P bytes of one step for one wave
  // vector-memory instructions issued after a P slot's loads before it is
  // read: the stage's 8 dY loads, then the other slot's P and dY loads
  constexpr int kAfterP = 8 + 2 * NBW + 8;
  __shared__ __attribute__((aligned(16))) unsigned char lds[acc_lds_bytes<NB16>()];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int rpart = wave / kLanes;  // r part of this wave
  const int wl = wave % kLanes;     // step lane of this wave
  const int m = lane & 15;   // A-operand row group (d columns)
  const int g4 = lane >> 4;  // which 8 tokens of the 32-token step
  const int task = xcd_runs((int)(blockIdx.y * gridDim.x + blockIdx.x),
                            (int)(gridDim.x * gridDim.y));
  const int sp = task / (int)gridDim.x;
  const int dgg = task % (int)gridDim.x;   // d group across outputs
  const OutSel out = select_out(tab, dgg, Pt1);
  const uint16_t* __restrict__ dY = out.dY;
  const int64_t ldd = out.ldd;
  const int d = out.d;
  float* __restrict__ S = out.S;
  const uint16_t* __restrict__ Pt = out.Pt;
  const int dg = dgg - out.dg_first;                                 // within the output
  const int dc0 = dg * DC;
  const int col = dc0 + Q * m;
  const int s_begin = sp * steps_per_split;
  const int s_end = min(steps_total, s_begin + steps_per_split);

  float acc[NREGW];
#pragma unroll
  for (int i = 0; i < NREGW; ++i) acc[i] = 0.0f;
  const int vo = dy_lane_offset(ldd, d, col, g4);
  const int qvalid = d - col;     // columns col + q < d are real (MASKED)

  unsigned char* ring = lds + wave * 2 * kSlot;
  auto p_issue = [&](int step, int slot) {
#pragma unroll
    for (int blk = 0; blk < 2 * NBW; ++blk) {
      const uint16_t* src =
          Pt + p_block(step, rpart * NBW + (blk >> 1), blk & 1, NB16) + 8 * lane;
      lds_dma16(src, lds_addr(ring + slot * kSlot + blk * 1024));
    }
  };
  // One step: Q A operands (d rows x tokens, transposed in registers with
  // v_perm from the row loads) against NBW hi/lo pairs of P operands.
  // mc: std::true_type in a work-group whose d group is ragged (the column
  // masks), std::false_type elsewhere; the pipeline below is instantiated
  // for both and each work-group runs one.
  auto mfma_step = [&](auto mc, const DyStage<Q>& ds, const u32x4& bh, const u32x4& bl,
                       int nb) {
    constexpr bool MC = decltype(mc)::value;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      // K assignment: lane group g4, element e <-> token tb + e.
      u32x4 a;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = __builtin_amdgcn_perm(ds.R[2 * u + 1][q >> 1], ds.R[2 * u][q >> 1],
                                     (q & 1) ? 0x07060302u : 0x05040100u);
      }
      if constexpr (MC) {
        if (q >= qvalid) a = u32x4{0u, 0u, 0u, 0u};   // column past d
      }
      const int i0 = (q * NBW + nb) * 4;
      f32x4 c4 = {acc[i0], acc[i0 + 1], acc[i0 + 2], acc[i0 + 3]};
      c4 = mfma16(a, bh, c4);
      c4 = mfma16(a, bl, c4);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i0 + v] = c4[v];
    }
  };
  auto compute_lds = [&](auto mc, const DyStage<Q>& ds, int slot) {
    const unsigned char* base = ring + slot * kSlot + 16 * lane;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const u32x4 bh = *reinterpret_cast<const u32x4*>(base + (2 * nb) * 1024);
      const u32x4 bl = *reinterpret_cast<const u32x4*>(base + (2 * nb + 1) * 1024);
      mfma_step(mc, ds, bh, bl, nb);
    }
  };

  // Ping-pong pipeline over this wave's n steps: the loads of step j + 1 are
  // in flight while step j is multiplied, and step j + 2 is issued into the
  // stage step j frees.  The dY loads of a stage are issued on every pass,
  // for steps past the wave's last as loads of zero bytes: every path into
  // the loop header then has the same loads outstanding, and the compiler's
  // own wait for a stage's dY registers leaves the other stage's loads in
  // flight (with a conditional reload it had to assume the stage just read
  // was the last one issued, and drained every load every two steps).  Only
  // the P copies, which the compiler does not see, are skipped past the last
  // step, so before reading a P slot the kernel waits for every load older
  // than the next step's: 8 dY loads, the next step's 2 NBW P copies when it
  // exists, and its 8 dY loads.  sched_barrier keeps the scheduler from
  // sinking loads back next to their consumers.
  const int first = s_begin + wl;
  const int n = first < s_end ? (s_end - first + kLanes - 1) / kLanes : 0;
  auto step_of = [&](int jj) { return first + kLanes * jj; };
  auto pipeline = [&](auto mc) {
    DyStage<Q> y0, y1;
    auto wait_slot = [&](int jj) {
      if (jj + 1 < n) vm_wait<kAfterP>();
      else vm_wait<16>();
    };
    auto stage = [&](int jj, int slot, DyStage<Q>& y) {
      const bool valid = jj < n;
      if (valid) p_issue(step_of(jj), slot);
      load_dy_stage<Q>(dY, ldd, T, vo, valid ? step_of(jj) : first, y, valid);
    };
    stage(0, 0, y0);
    stage(1, 1, y1);
    __builtin_amdgcn_sched_barrier(0);
    for (int jj = 0; jj < n; jj += 2) {
      wait_slot(jj);
      compute_lds(mc, y0, 0);
      __builtin_amdgcn_sched_barrier(0);
      lgkm_wait0();
      stage(jj + 2, 0, y0);
      __builtin_amdgcn_sched_barrier(0);
      if (jj + 1 < n) {
        wait_slot(jj + 1);
        compute_lds(mc, y1, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      lgkm_wait0();
      stage(jj + 3, 1, y1);
      __builtin_amdgcn_sched_barrier(0);
    }
    vm_wait<0>();   // the ring is reused below
  };
  if (n > 0) {
    if (MASKED && dc0 + DC > d)
      pipeline(std::true_type{});
    else
      pipeline(std::false_type{});
  }

  // Sum over the waves that share an r part, in a fixed order (((l0 + l1) +
  // l2) + ...), CH registers per round through LDS as 16-byte quads (four
  // registers of one lane); each wave sums its share of the round's quads
  // and writes them out: to the partial tile of this split (register-major,
  // coalesced) or, with a single split, into S.
  static_assert(CH % 4 == 0 && NREGW % CH == 0, "whole quads and rounds");
  constexpr int CQ = CH / 4;                                   // quads per round
  constexpr int kPerQ = CQ / kLanes > 0 ? CQ / kLanes : 1;     // quads per wave
  f32x4* red = reinterpret_cast<f32x4*>(lds);
  float* my = part ? part + ((int64_t)sp * gridDim.x + dgg) * (NREG * 64) : nullptr;
  __syncthreads();
#pragma unroll
  for (int c0 = 0; c0 < NREGW; c0 += CH) {
    // wave register c0 + 4 jq + e = (q NBW + nb) 4 + e -> tile register
    auto tile_reg = [&](int jq, int e) {
      const int lr = c0 + 4 * jq + e;
      const int q = lr / (NBW * 4);
      const int rem = lr % (NBW * 4);
      return (q * NB16 + rpart * NBW + (rem >> 2)) * 4 + (rem & 3);
    };
    // earlier deferred contributions of this split, loaded while the round
    // goes through LDS
    float old[kPerQ][4];
    if (my && tab.pending) {
#pragma unroll
      for (int u = 0; u < kPerQ; ++u) {
        const int jq = wl * kPerQ + u;
#pragma unroll
        for (int e = 0; e < 4; ++e) old[u][e] = jq < CQ ? my[tile_reg(jq, e) * 64 + lane] : 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < CQ; ++j)
      red[(wave * CQ + j) * 64 + lane] =
          f32x4{acc[c0 + 4 * j], acc[c0 + 4 * j + 1], acc[c0 + 4 * j + 2], acc[c0 + 4 * j + 3]};
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPerQ; ++u) {
      const int jq = wl * kPerQ + u;           // quad within the round
      if (jq < CQ) {
        const int base = rpart * kLanes;       // first wave of this r part
        f32x4 v = red[(base * CQ + jq) * 64 + lane];
#pragma unroll
        for (int w = 1; w < kLanes; ++w) v += red[((base + w) * CQ + jq) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = tile_reg(jq, e);
          if (my) {
            my[i * 64 + lane] = tab.pending ? old[u][e] + v[e] : v[e];
          } else {
            const int drow = acc_drow<Q, NB16>(dc0, i, lane);
            const int rc = acc_rcol<NB16>(i, lane);
            if (drow < d && rc < r) {
              float* sp_ = S + (int64_t)drow * r + rc;
              *sp_ = tab.overwrite ? v[e] : *sp_ + v[e];
            }
          }
        }
      }
    }
    if (c0 + CH < NREGW) __syncthreads();   // the next round overwrites the buffer
  }
}

// S += dY^T P for r = 128 and 256, where accumulate_kernel's waves split r
// and each loads the same dY rows and its own P tiles: at r = 256 that moves
// ~128 KB through a CU's vector-memory path per 2048 matrix-core cycles, about
// all it takes, and the matrix cores sat ~50 % busy.  Here a work-group owns
// DP = 8 / (r / 64) d groups of 128 columns and all of r over a range of
// 32-token steps; wave w takes d group w % DP and r columns 64 (w / DP) ..
// + 63 (128 x 64 accumulators, as in accumulate_kernel).  Per step the dY
// rows of all DP groups (32 x 128 DP bf16) and the P tile of all r reach LDS
// once, by direct global->LDS copies spread over the waves, and every wave
// reads its operands from there: 48 KB per step per work-group for 2048
// matrix-core cycles per SIMD.  Three stages: a step's copies are issued two
// steps ahead, one barrier per step.  No cross-wave sum: each wave writes its
// own 128 x 64 block (partial tile or S).
template <int NB16, bool MASKED, class Tab>
__global__ __launch_bounds__(512) void accumulate_wide_kernel(
    Tab tab, int T, int r, const uint16_t* __restrict__ Pt1, int steps_total, int steps_per_split,
    int n_dgroups, float* __restrict__ part) {
  constexpr int Q = 8;
  constexpr int NBW = 4;                     // 16-column r blocks per wave
  constexpr int RPW = NB16 / NBW;            // waves along r
  constexpr int DP = kAccWaves / RPW;        // d groups per work-group
  constexpr int NREG = Q * NB16 * 4;         // registers of a d group's tile
  constexpr int NREGW = Q * NBW * 4;         // accumulators per lane
  constexpr int kDyRow = DP * 16 * Q * 2;    // bytes of one token row of the dY tile
  constexpr int kDyBytes = 32 * kDyRow;
  constexpr int kPBytes = NB16 * 2 * 1024;   // one step of P, every r block, hi and lo
  constexpr int kStage = kDyBytes + kPBytes;
  constexpr int kStages = 3;
  constexpr int kCopies = kStage / 1024;     // 1 KB copies per step
  constexpr int kCopiesW = kCopies / kAccWaves;
  static_assert(kCopies % kAccWaves == 0, "copies spread evenly over the waves");
  static_assert(kStages * kStage <= 160 * 1024, "stages fit in LDS");
  __shared__ __attribute__((aligned(16))) unsigned char lds[kStages * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dpart = wave % DP;
  const int rpart = wave / DP;
  const int m = lane & 15;
  const int g4 = lane >> 4;
  const int task = xcd_runs((int)(blockIdx.y * gridDim.x + blockIdx.x),
                            (int)(gridDim.x * gridDim.y));
  const int sp = task / (int)gridDim.x;
  const int wg = task % (int)gridDim.x;
  // output of this work-group (wave-uniform compares on the table)
  const OutSel out = select_out_wg(tab, wg, Pt1);
  const uint16_t* dY = out.dY;
  const int64_t ldd = out.ldd;
  const int d = out.d;
  float* S = out.S;
  const uint16_t* __restrict__ Pt = out.Pt;
  const int dg_first = out.dg_first, dg_end = out.dg_end, wg_first = out.wg_first;
  const int col_wg = (wg - wg_first) * DP * 16 * Q;   // first d column of the work-group
  const int dg_local = (wg - wg_first) * DP + dpart;   // this wave's d group in the output
  const bool group_ok = dg_first + dg_local < dg_end;
  const int dc0 = dg_local * 16 * Q;
  const int s_begin = sp * steps_per_split;
  const int s_end = min(steps_total, s_begin + steps_per_split);
  const int n = s_end - s_begin;
  // the masks and clamps matter only on the ragged last step and in
  // work-groups that reach past d
  const bool cols_edge = MASKED && col_wg + DP * 16 * Q > d;

  // Copies of step `step` into stage st: copy c = j * 8 + wave; the first
  // kDyBytes / 1 KB copies bring dY (row-major, kDyRow bytes per token row;
  // rows past T re-read row T - 1 and columns past d the row's first 8, both
  // cleared by clear_edges), the rest the step's P blocks (contiguous).
  auto issue = [&](int step, int st) {
    unsigned char* base = lds + st * kStage;
#pragma unroll
    for (int j = 0; j < kCopiesW; ++j) {
      const int c = j * kAccWaves + wave;
      if (c < kDyBytes / 1024) {
        const int b = c * 1024 + 16 * lane;
        int t = step * 32 + b / kDyRow;
        int col = col_wg + (b % kDyRow) / 2;
        if (MASKED && (step + 1) * 32 > T) t = t < T ? t : T - 1;   // ragged last step only
        if (cols_edge) col = col < d ? col : 0;
        lds_dma16((const void*)(dY + (int64_t)t * ldd + col), lds_addr(base + c * 1024));
      } else {
        const int cp = c - kDyBytes / 1024;
        lds_dma16((const void*)(Pt + p_block(step, 0, 0, NB16) + cp * 512 + 8 * lane),
                  lds_addr(base + kDyBytes + cp * 1024));
      }
    }
  };

  float acc[NREGW];
#pragma unroll
  for (int i = 0; i < NREGW; ++i) acc[i] = 0.0f;

  // On an edge step (the ragged last step, or any step of a work-group that
  // reaches past d) the staged dY tile gets its rows past T and columns past
  // d cleared in LDS, by all threads between two barriers, so compute never
  // masks.  Pieces wholly inside are left alone.
  auto clear_edges = [&](int step, int st) {
    unsigned char* base = lds + st * kStage;
    for (int p = tid; p < kDyBytes / 16; p += 64 * kAccWaves) {
      const int row = p / (kDyRow / 16);
      const int piece = p % (kDyRow / 16);
      const int valid = step * 32 + row < T ? d - (col_wg + 8 * piece) : 0;
      if (valid < 8) {
        u32x4* q4 = reinterpret_cast<u32x4*>(base + p * 16);
        *q4 = *q4 & keep_mask8(valid);
      }
    }
  };

  auto compute = [&](int st) {
    const unsigned char* base = lds + st * kStage;
    // dY rows 8 g4 + e of the step, columns dc0 + Q m .. + 7 (as
    // load_dy_stage gives them), and the wave's P operands
    u32x4 row[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      row[e] = *reinterpret_cast<const u32x4*>(base + (8 * g4 + e) * kDyRow + dpart * 256 +
                                               16 * m);
    u32x4 bh[NBW], bl[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int nbg = rpart * NBW + nb;
      bh[nb] = *reinterpret_cast<const u32x4*>(base + kDyBytes + (2 * nbg) * 1024 + 16 * lane);
      bl[nb] = *reinterpret_cast<const u32x4*>(base + kDyBytes + (2 * nbg + 1) * 1024 + 16 * lane);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      u32x4 a;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        a[u] = __builtin_amdgcn_perm(row[2 * u + 1][q >> 1], row[2 * u][q >> 1],
                                     (q & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int i0 = (q * NBW + nb) * 4;
        f32x4 c4 = {acc[i0], acc[i0 + 1], acc[i0 + 2], acc[i0 + 3]};
        c4 = mfma16(a, bh[nb], c4);
        c4 = mfma16(a, bl[nb], c4);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i0 + v] = c4[v];
      }
    }
  };

  if (n > 0) {
    issue(s_begin, 0);
    if (n > 1) issue(s_begin + 1, 1);
    for (int j = 0; j < n; ++j) {
      // this wave's copies of step j are done (only step j + 1's may be
      // outstanding), then everybody's; stage (j + 2) % 3, refilled below,
      // was last read in step j - 1, which every wave has finished
      if (j + 1 < n) vm_wait<kCopiesW>();
      else vm_wait<0>();
      __syncthreads();
      if (MASKED && (cols_edge || (s_begin + j + 1) * 32 > T)) {   // work-group uniform
        clear_edges(s_begin + j, j % kStages);
        __syncthreads();
      }
      // multiply first, then issue step j + 2's copies (measured 1-4 %
      // faster than issuing them ahead of the MFMAs)
      compute(j % kStages);
      if (j + 2 < n) issue(s_begin + j + 2, (j + 2) % kStages);
    }
  }
  if (!group_ok) return;

  // Wave register il = (q NBW + nb) 4 + e -> tile register of its d group.
  const int dgg = dg_first + dg_local;
  float* my = part ? part + ((int64_t)sp * n_dgroups + dgg) * (NREG * 64) : nullptr;
#pragma unroll
  for (int il = 0; il < NREGW; ++il) {
    const int q = il / (NBW * 4);
    const int rem = il % (NBW * 4);
    const int i = (q * NB16 + rpart * NBW + (rem >> 2)) * 4 + (rem & 3);
    const float v = acc[il];
    if (my) {
      my[i * 64 + lane] = tab.pending ? my[i * 64 + lane] + v : v;
    } else {
      const int drow = acc_drow<Q, NB16>(dc0, i, lane);
      const int rc = acc_rcol<NB16>(i, lane);
      if (drow < d && rc < r) {
        float* sp_ = S + (int64_t)drow * r + rc;
        *sp_ = tab.overwrite ? v : *sp_ + v;
      }
    }
  }
}

// S += sum over splits of the partial tiles, in split order.  One thread per
// four consecutive floats of a tile (four lanes with the same d row and four
// consecutive r columns).
template <int Q, int NB16, class Tab>
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ part,
                                                       int n_split, int n_dgroups, Tab tab,
                                                       int r) {
  constexpr int NREG = Q * NB16 * 4;
  constexpr int TILE = NREG * 64;
  const int64_t idx4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_split = (int64_t)n_dgroups * TILE;
  if (idx4 * 4 >= per_split) return;
  const int64_t flat = idx4 * 4;
  const int dgg = (int)(flat / TILE);
  const OutSel out = select_out(tab, dgg, nullptr);
  const int within = (int)(flat % TILE);
  const int i = within >> 6;
  const int ln = within & 63;       // multiple of 4
  const int drow = acc_drow<Q, NB16>((dgg - out.dg_first) * 16 * Q, i, ln);
  const int rc = acc_rcol<NB16>(i, ln);
  if (drow >= out.d) return;
  float* srow = out.S + (int64_t)drow * r;
  // float4 access when r % 4 == 0 and S is 16-byte aligned
  const bool vec = (r % 4) == 0 && (reinterpret_cast<uintptr_t>(out.S) & 15) == 0 && rc + 4 <= r;
  // Loads go out eight splits at a time (with S in the first group), so one
  // memory latency covers each group; the adds still run in split order.
  // Slots past the last split re-read it and are not added.
  constexpr int G = 8;
  const bool add = !tab.overwrite;
  f32x4 sv = {0.f, 0.f, 0.f, 0.f};
  if (vec && add) sv = *reinterpret_cast<const f32x4*>(srow + rc);
  const float* pp = part + flat;
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < n_split; sp += G) {
    f32x4 v[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int su = sp + u < n_split ? sp + u : n_split - 1;
      v[u] = *reinterpret_cast<const f32x4*>(pp + (int64_t)su * per_split);
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (sp + u < n_split) sum += v[u];
    }
  }
  if (vec) {
    *reinterpret_cast<f32x4*>(srow + rc) = sv + sum;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (rc + e < r) srow[rc + e] = add ? srow[rc + e] + sum[e] : sum[e];
  }
}

// Kernel-choice overrides set through logra_set_kernel_choice (tests and
// measurements): -1 automatic, 0 never, 1 always (for the projection tile, 2:
// always, with 128-token tiles from r = 128).
std::atomic<int> g_choice_project_tile{-1};
std::atomic<int> g_choice_acc_wide{-1};

// The token blocks per work-group of project_tile_kernel for this call, or 0
// for project_kernel (the tile needs two 32-row blocks of A, its 128-token
// form four).  The tile builds each basis operand for two or four token
// blocks, which pays wherever operand building bounds project_kernel: always
// for the Gaussian basis, and for the sign basis once its work-groups still
// fill all 256 CUs (below that, project_kernel's more work-groups are worth
// more); the 128-token form wherever its work-groups, all groups together,
// fill them.
int tile_blocks(const SketchPlan& p, int nb32, bool gauss) {
  if (nb32 < 2) return 0;
  const int tb4 = nb32 >= 4 ? 4 : 2;
  const int mode = g_choice_project_tile.load(std::memory_order_relaxed);
  if (mode == 0) return 0;
  if (mode == 1) return 2;
  if (mode == 2) return tb4;
  if (nb32 >= 4 && p.n_groups * ((p.t_pad + 127) / 128) >= 256) return 4;
  return gauss || p.t_pad / 64 >= 256 ? 2 : 0;
}

// Groups and their block count in a projection launch.
inline int proj_groups(const ProjOne&) { return 1; }
inline int proj_groups(const ProjTable& t) { return t.n; }
inline bool proj_masked(const ProjOne& t) { return (t.k % 256) != 0; }
inline bool proj_masked(const ProjTable& t) {
  bool m = false;
  for (int g = 0; g < t.n; ++g) m = m || (t.k[g] % 256) != 0;
  return m;
}
inline void set_blocks(ProjOne&, int) {}
inline void set_blocks(ProjTable& t, int n_blk) { t.n_blk = n_blk; }

template <int NB, bool GAUSS, bool MASKED, class PT>
void launch_project_t(const SketchPlan& p, const PT& tab, int T, float c, hipStream_t s) {
  constexpr int W = proj_waves(NB);
  const dim3 grid((unsigned)(proj_groups(tab) * (p.t_pad / 32)));
  hipLaunchKernelGGL((project_kernel<NB, GAUSS, MASKED, W, PT>), grid, dim3(64 * W), 0, s, tab, T,
                     p.rp, c);
}

// One launch over every group's token blocks.  MASKED (a ragged last chunk of
// k) when any group's k is not a multiple of 256; the kernels test the edge
// per chunk, so groups with whole chunks run as without the mask.
template <int NB, class PT>
hipError_t launch_project(const SketchPlan& p, PT tab, int T, bool gauss, float c, hipStream_t s) {
  const bool masked = proj_masked(tab);
  if constexpr (NB >= 2) {
    const int tb = tile_blocks(p, NB, gauss);
    if (tb > 0) {
      const int n_blk = (int)((p.t_pad + 32 * tb - 1) / (32 * tb));
      set_blocks(tab, n_blk);
      const dim3 grid((unsigned)(proj_groups(tab) * n_blk));
      const float cc = gauss ? 1.0f : c;
#define LOGRA_TILE(G, M, TB)                                                                     \
  hipLaunchKernelGGL((project_tile_kernel<NB / TB, G, M, TB, PT>), grid, dim3(512), 0, s, tab, T, \
                     p.rp, p.steps, cc)
#define LOGRA_TILES(TB)                         \
  if (gauss) {                                  \
    if (masked) LOGRA_TILE(true, true, TB);     \
    else LOGRA_TILE(true, false, TB);           \
  } else {                                      \
    if (masked) LOGRA_TILE(false, true, TB);    \
    else LOGRA_TILE(false, false, TB);          \
  }
      if constexpr (NB >= 4) {
        if (tb == 4) {
          LOGRA_TILES(4)
          return hipGetLastError();
        }
      }
      LOGRA_TILES(2)
#undef LOGRA_TILES
#undef LOGRA_TILE
      return hipGetLastError();
    }
  }
  set_blocks(tab, (int)(p.t_pad / 32));
  if (gauss) {
    if (masked) launch_project_t<NB, true, true>(p, tab, T, 1.0f, s);
    else launch_project_t<NB, true, false>(p, tab, T, 1.0f, s);
  } else {
    if (masked) launch_project_t<NB, false, true>(p, tab, T, c, s);
    else launch_project_t<NB, false, false>(p, tab, T, c, s);
  }
  return hipGetLastError();
}

template <int Q, int NB16, class Tab>
hipError_t launch_finalize(const SketchPlan& p, const Tab& tab, int r, float* part,
                           hipStream_t s) {
  const int64_t quads = (int64_t)p.n_dgroups * Q * NB16 * 4 * 64 / 4;
  hipLaunchKernelGGL((finalize_kernel<Q, NB16, Tab>), dim3((unsigned)((quads + 255) / 256)),
                     dim3(256), 0, s, part, p.n_split, p.n_dgroups, tab, r);
  return hipGetLastError();
}

// Partial tiles are used with several splits, and for every call of a
// deferred chain (defer: keep the result there; tab.pending: add to them).
// Pt1: the P of a one-group call (an OutTable); a LayerOutTable carries each
// output's own.
template <int Q, int NB16, class Tab>
hipError_t launch_accumulate(const SketchPlan& p, const Tab& tab, int T, int r,
                             const uint16_t* Pt1, float* part, bool defer, hipStream_t s) {
  const dim3 grid((unsigned)p.n_dgroups, (unsigned)p.n_split);
  float* pp = p.n_split > 1 || defer || tab.pending ? part : nullptr;
  // masked for a ragged d group only: rows past T read as zero through the
  // buffer loads whatever the template
  bool masked = false;
  for (int o = 0; o < tab.n; ++o) masked = masked || (tab.d[o] % (16 * Q)) != 0;
  if (masked) {
    hipLaunchKernelGGL((accumulate_kernel<Q, NB16, true, Tab>), grid, dim3(64 * kAccWaves), 0, s,
                       tab, T, r, Pt1, p.steps, p.steps_per_split, pp);
  } else {
    hipLaunchKernelGGL((accumulate_kernel<Q, NB16, false, Tab>), grid, dim3(64 * kAccWaves), 0, s,
                       tab, T, r, Pt1, p.steps, p.steps_per_split, pp);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pp == nullptr || defer) return e;
  return launch_finalize<Q, NB16>(p, tab, r, part, s);
}

template <int NB16, class Tab>
hipError_t launch_accumulate_wide(const SketchPlan& p, const Tab& tab, int T, int r,
                                  const uint16_t* Pt1, float* part, bool defer, hipStream_t s) {
  constexpr int DP = kAccWaves / (NB16 / 4);
  const dim3 grid((unsigned)p.n_wg, (unsigned)p.n_split);
  float* pp = p.n_split > 1 || defer || tab.pending ? part : nullptr;
  // masked: a ragged step, a ragged d group, or a work-group whose last d
  // groups lie past its output (their columns must not be read)
  bool masked = (T % 32) != 0;
  for (int o = 0; o < tab.n; ++o)
    masked = masked || (tab.d[o] % (16 * kAccQ)) != 0 ||
             ((tab.dg_off[o + 1] - tab.dg_off[o]) % DP) != 0;
  if (masked) {
    hipLaunchKernelGGL((accumulate_wide_kernel<NB16, true, Tab>), grid, dim3(64 * kAccWaves), 0, s,
                       tab, T, r, Pt1, p.steps, p.steps_per_split, p.n_dgroups, pp);
  } else {
    hipLaunchKernelGGL((accumulate_wide_kernel<NB16, false, Tab>), grid, dim3(64 * kAccWaves), 0,
                       s, tab, T, r, Pt1, p.steps, p.steps_per_split, p.n_dgroups, pp);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pp == nullptr || defer) return e;
  return launch_finalize<kAccQ, NB16>(p, tab, r, part, s);
}

// The projection and accumulate launches of one call with the given tables.
// The projection launch of a call (P for every input group of the table).
template <class PT>
hipError_t launch_project_phase(const SketchPlan& p, const PT& pt, int T, bool gauss, float c,
                                hipStream_t s) {
  switch (p.nb32) {
    case 1: return launch_project<1>(p, pt, T, gauss, c, s);
    case 2: return launch_project<2>(p, pt, T, gauss, c, s);
    case 4: return launch_project<4>(p, pt, T, gauss, c, s);
    default: return launch_project<8>(p, pt, T, gauss, c, s);
  }
}

// The accumulate launch (and, unless deferred, the split reduction) of a call.
template <class Tab>
hipError_t launch_accumulate_phase(const SketchPlan& p, const Tab& tab, const uint16_t* Pt1, int T,
                                   int r, bool defer, float* part, hipStream_t s) {
  if (p.acc_wide) {
    if (p.rp == 128) return launch_accumulate_wide<8>(p, tab, T, r, Pt1, part, defer, s);
    return launch_accumulate_wide<16>(p, tab, T, r, Pt1, part, defer, s);
  }
  switch (p.rp) {
    case 16: return launch_accumulate<kAccQ, 1>(p, tab, T, r, Pt1, part, defer, s);
    case 32: return launch_accumulate<kAccQ, 2>(p, tab, T, r, Pt1, part, defer, s);
    case 64: return launch_accumulate<kAccQ, 4>(p, tab, T, r, Pt1, part, defer, s);
    case 128: return launch_accumulate<kAccQ, 8>(p, tab, T, r, Pt1, part, defer, s);
    default: return launch_accumulate<kAccQ, 16>(p, tab, T, r, Pt1, part, defer, s);
  }
}

template <class PT, class Tab>
hipError_t launch_tables(const SketchPlan& p, const PT& pt, const Tab& tab, const uint16_t* Pt1,
                         int T, int r, bool gauss, float c, bool defer, float* part,
                         hipStream_t s) {
  const hipError_t e = launch_project_phase(p, pt, T, gauss, c, s);
  if (e != hipSuccess) return e;
  return launch_accumulate_phase(p, tab, Pt1, T, r, defer, part, s);
}

// The output fields shared by both table types.
template <class Tab>
void fill_outputs(Tab& tab, const SketchPlan& p, const SketchOut* outs, bool overwrite,
                  bool pending) {
  tab.n = p.n_out;
  tab.overwrite = overwrite ? 1 : 0;
  tab.pending = pending ? 1 : 0;
  for (int o = 0; o <= p.n_out; ++o) {
    tab.dg_off[o] = p.dg_off[o];
    tab.wg_off[o] = p.wg_off[o];
  }
  for (int o = 0; o < p.n_out; ++o) {
    tab.dY[o] = outs[o].dY;
    tab.ldd[o] = outs[o].ldd;
    tab.d[o] = (int)outs[o].d;
    tab.S[o] = outs[o].S;
  }
}

}  // namespace

bool make_sketch_plan_groups(int64_t T, int n_groups, const int64_t* k, const int* n_out_g,
                             const int64_t* d, int r, SketchPlan* p) {
  if (T < 0 || T >= (int64_t(1) << 31) || r < 1 || r > 256) return false;
  if (n_groups < 1 || n_groups > kMaxGroups) return false;
  SketchPlan q{};
  q.n_groups = n_groups;
  int n_out = 0;
  for (int g = 0; g < n_groups; ++g) {
    if (k[g] < 1 || k[g] >= (int64_t(1) << 31)) return false;
    if (n_out_g[g] < 1 || n_out_g[g] > kMaxShared) return false;
    q.k_pad[g] = round_up(k[g], 256);
    q.out_off[g] = n_out;
    n_out += n_out_g[g];
  }
  if (n_out > kMaxOut) return false;
  q.out_off[n_groups] = n_out;
  q.rp = r <= 16 ? 16 : r <= 32 ? 32 : r <= 64 ? 64 : r <= 128 ? 128 : 256;
  q.p_rows = q.rp < 32 ? 32 : q.rp;
  q.nb32 = q.p_rows / 32;
  q.q_cols = kAccQ;
  q.t_pad = round_up(T > 0 ? T : 1, 32);
  q.steps = (int)(q.t_pad / 32);
  const int dc = 16 * q.q_cols;
  q.n_out = n_out;
  // The wide kernel from r = 128 once T gives each work-group enough steps
  // (T >= 16384): at T = 8192 it left CUs idle and measured slower.
  const int wide_mode = g_choice_acc_wide.load(std::memory_order_relaxed);
  q.acc_wide = q.rp >= 128 && (wide_mode >= 0 ? wide_mode == 1 : q.steps >= 512);
  q.wg_groups = q.acc_wide ? kAccWaves / (q.rp / 64) : 1;
  int64_t groups = 0, wgs_d = 0;
  for (int o = 0; o < n_out; ++o) {
    if (d[o] < 1 || d[o] >= (int64_t(1) << 31)) return false;
    q.dg_off[o] = (int)groups;
    q.wg_off[o] = (int)wgs_d;
    const int64_t g = (d[o] + dc - 1) / dc;
    groups += g;
    wgs_d += (g + q.wg_groups - 1) / q.wg_groups;
  }
  if (groups >= (int64_t(1) << 27)) return false;   // finalize grid: 8 per group
  q.dg_off[n_out] = (int)groups;
  q.wg_off[n_out] = (int)wgs_d;
  q.n_dgroups = (int)groups;
  q.n_wg = (int)wgs_d;
  // Work-groups along T: at most so many that each wave keeps two 32-token
  // steps; among those counts, the one with the least modelled cost: the dY
  // stream slowed by the share of the 256 CUs that the work-groups' rounds
  // leave idle (one work-group per CU), plus writing and reading the split
  // partial tiles and the split-reduction launch (~25 MB of streaming).
  // (The wide kernel's waves all take every step of their split: at least
  // four steps each, so the three-stage copy ring fills.)
  const int lanes = kAccWaves / acc_rsplit(q.rp / 16);   // waves along the steps
  const int min_steps = q.acc_wide ? 4 : 2 * lanes;
  const int max_split = q.steps / min_steps > 0 ? q.steps / min_steps : 1;
  const double dy_bytes = 2.0 * (double)q.t_pad * (double)groups * dc;
  const int64_t wgs_along_d = q.acc_wide ? wgs_d : groups;
  int n_split = 1;
  double best = 0.0;
  for (int ns = 1; ns <= max_split && ns <= 64; ++ns) {
    const int64_t wgs = wgs_along_d * ns;
    const double eff = (double)wgs / (double)(((wgs + 255) / 256) * 256);
    const double cost = dy_bytes / eff +
                        (ns > 1 ? 8.0 * ns * (double)groups * dc * q.rp + 25e6 : 0.0);
    if (ns == 1 || cost < best * 0.999) {
      best = cost;
      n_split = ns;
    }
  }
  q.steps_per_split = (q.steps + n_split - 1) / n_split;
  q.n_split = (q.steps + q.steps_per_split - 1) / q.steps_per_split;
  q.d_pad = (int64_t)q.n_dgroups * dc;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  for (int g = 0; g < n_groups; ++g) q.off_pt[g] = take(plan_p_bytes(q));
  // (one split's worth even when a single split writes S directly: a
  // deferred call keeps its result there)
  q.off_part = take(plan_part_bytes(q));
  for (int g = 0; g < n_groups; ++g) q.off_gauss[g] = take(plan_gauss_bytes(q, g));
  q.total = off;
  *p = q;
  return true;
}

bool set_kernel_choice(int which, int mode) {
  if (mode < -1 || mode > (which == 0 ? 2 : 1)) return false;
  if (which == 0) g_choice_project_tile.store(mode, std::memory_order_relaxed);
  else if (which == 1) g_choice_acc_wide.store(mode, std::memory_order_relaxed);
  else return false;
  return true;
}

hipError_t launch_sketch(const SketchPlan& p, const SketchGroup* groups, const SketchOut* outs,
                         int T, int r, int kind, bool overwrite, bool defer, bool pending,
                         char* ws, hipStream_t s) {
  float* part = reinterpret_cast<float*>(ws + p.off_part);
  const bool gauss = kind == 1;
  const float c = sign_scale(r);
  for (int g = 0; g < p.n_groups; ++g) {
    if (!gauss) break;
    const int64_t threads = (int64_t)p.p_rows * (p.k_pad[g] >> 2);
    hipLaunchKernelGGL(gauss_basis_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       s, groups[g].seed, groups[g].stream, r, (int)groups[g].k, p.p_rows,
                       p.k_pad[g], c, reinterpret_cast<uint16_t*>(ws + p.off_gauss[g]));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.n_groups == 1) {
    const SketchGroup& gr = groups[0];
    uint16_t* Pt = reinterpret_cast<uint16_t*>(ws + p.off_pt[0]);
    const ProjOne pt{gr.X, gr.ldx, (int)gr.k, gr.seed, gr.stream,
                     reinterpret_cast<const uint16_t*>(ws + p.off_gauss[0]), p.k_pad[0], Pt};
    OutTable tab{};
    fill_outputs(tab, p, outs, overwrite, pending);
    return launch_tables(p, pt, tab, Pt, T, r, gauss, c, defer, part, s);
  }
  // Projection table: groups with the largest k first, so the longest
  // work-groups are dispatched first and the short ones fill in behind them.
  int order[kMaxGroups];
  for (int g = 0; g < p.n_groups; ++g) order[g] = g;
  for (int a = 1; a < p.n_groups; ++a)
    for (int b = a; b > 0 && groups[order[b]].k > groups[order[b - 1]].k; --b) {
      const int t = order[b];
      order[b] = order[b - 1];
      order[b - 1] = t;
    }
  ProjTable pt{};
  pt.n = p.n_groups;
  for (int j = 0; j < p.n_groups; ++j) {
    const int g = order[j];
    const SketchGroup& gr = groups[g];
    pt.X[j] = gr.X;
    pt.ldx[j] = gr.ldx;
    pt.k[j] = (int)gr.k;
    pt.seed[j] = gr.seed;
    pt.stream[j] = gr.stream;
    pt.Ab[j] = reinterpret_cast<const uint16_t*>(ws + p.off_gauss[g]);
    pt.lda[j] = p.k_pad[g];
    pt.Pt[j] = reinterpret_cast<uint16_t*>(ws + p.off_pt[g]);
  }
  LayerOutTable tab{};
  fill_outputs(tab, p, outs, overwrite, pending);
  for (int g = 0; g < p.n_groups; ++g)
    for (int o = p.out_off[g]; o < p.out_off[g + 1]; ++o)
      tab.Pt[o] = reinterpret_cast<const uint16_t*>(ws + p.off_pt[g]);
  return launch_tables(p, pt, tab, nullptr, T, r, gauss, c, defer, part, s);
}

hipError_t launch_project_only(const SketchPlan& p, const SketchGroup& g, int T, int r, int kind,
                               uint16_t* P, uint16_t* gauss_ws, hipStream_t s) {
  const bool gauss = kind == 1;
  const float c = sign_scale(r);
  if (gauss) {
    const int64_t threads = (int64_t)p.p_rows * (p.k_pad[0] >> 2);
    hipLaunchKernelGGL(gauss_basis_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       s, g.seed, g.stream, r, (int)g.k, p.p_rows, p.k_pad[0], c, gauss_ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const ProjOne pt{g.X, g.ldx, (int)g.k, g.seed, g.stream, gauss_ws, p.k_pad[0], P};
  return launch_project_phase(p, pt, T, gauss, c, s);
}

hipError_t launch_accumulate_only(const SketchPlan& p, const uint16_t* P, const SketchOut* outs,
                                  int T, int r, bool overwrite, bool defer, bool pending,
                                  float* part, hipStream_t s) {
  OutTable tab{};
  fill_outputs(tab, p, outs, overwrite, pending);
  return launch_accumulate_phase(p, tab, P, T, r, defer, part, s);
}

// S = 0, four floats per thread where the row allows (S of every output is
// a contiguous d x r array; its base is only 4-byte aligned).
__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ S, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n && (reinterpret_cast<uintptr_t>(S) & 15) == 0) {
    *reinterpret_cast<f32x4*>(S + i) = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    for (int64_t j = i; j < i + 4 && j < n; ++j) S[j] = 0.0f;
  }
}

hipError_t launch_zero_outputs(const SketchOut* outs, int n_out, int r, hipStream_t s) {
  if (n_out < 0 || n_out > kMaxOut) return hipErrorInvalidValue;
  for (int o = 0; o < n_out; ++o) {
    const int64_t n = outs[o].d * (int64_t)r;
    const int64_t blocks = (n + 1023) / 1024;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, outs[o].S, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace logra
