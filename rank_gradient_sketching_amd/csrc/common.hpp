// Device helpers shared by the gfx950 kernels of the LoGRA hot path.
//
// Sources:
//   [SALMON11] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
//              as 1, 2, 3", SC'11 - the Philox4x64 counter-based generator.
//   [LoGRA]    wispaper.ai summary of "LoGRA: Scaling LLM Reinforcement
//              Learning with Low-Rank Gradient Sketches", section Sketch: the
//              default projection entries are random signs scaled by
//              1/sqrt(r); section Sync: A is rebuilt from the seed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace logra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- Philox
// Philox4x64 with 10 rounds [SALMON11].  Each round multiplies words 0 and 2
// by fixed odd constants to 128-bit products and mixes the halves with words
// 1 and 3 and the key; the key advances by the Weyl increments between rounds.
constexpr uint64_t kPhiloxMul0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxMul1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxWeyl0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxWeyl1 = 0xBB67AE8584CAA73Bull;

struct Words4 {
  uint64_t w[4];
};

// Full 128-bit product of a constant a and b from four 32x32 -> 64 multiply-
// adds (v_mad_u64_u32); no partial sum can overflow 64 bits.
__device__ __forceinline__ void mulhilo64(uint64_t a, uint64_t b, uint64_t& hi,
                                          uint64_t& lo) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
  const uint32_t b0 = (uint32_t)b, b1 = (uint32_t)(b >> 32);
  const uint64_t p00 = (uint64_t)a0 * b0;
  const uint64_t p01 = (uint64_t)a0 * b1 + (p00 >> 32);
  const uint64_t p10 = (uint64_t)a1 * b0 + (uint32_t)p01;
  hi = (uint64_t)a1 * b1 + (p01 >> 32) + (p10 >> 32);
  lo = (p10 << 32) | (uint32_t)p00;
}

__device__ __forceinline__ Words4 philox4x64_10(uint64_t c0, uint64_t c1,
                                                uint64_t c2, uint64_t c3,
                                                uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round) {
      k0 += kPhiloxWeyl0;
      k1 += kPhiloxWeyl1;
    }
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(kPhiloxMul0, c0, hi0, lo0);
    mulhilo64(kPhiloxMul1, c2, hi1, lo1);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  Words4 out;
  out.w[0] = c0;
  out.w[1] = c1;
  out.w[2] = c2;
  out.w[3] = c3;
  return out;
}

// Sign block of row i, 256-column group g of the sign basis: bit b of word q
// is the sign of column 256 g + 64 q + b (set = negative).
__device__ __forceinline__ Words4 sign_block(uint64_t seed, uint64_t stream,
                                             uint64_t group, uint64_t row) {
  return philox4x64_10(group, row, 0, 0, seed, stream);
}

// Gaussian block of row i, 4-column group q: four standard normals by
// Box-Muller from the four output words (each gives a 24-bit uniform in (0,1)).
__device__ __forceinline__ void gaussian_block(uint64_t seed, uint64_t stream,
                                               uint64_t group, uint64_t row,
                                               float z[4]) {
  const Words4 b = philox4x64_10(group, row, 1, 0, seed, stream);
  float u[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    // (2 (w >> 41) + 1) < 2^24, so both the integer and the scaling are exact.
    u[a] = (float)(uint32_t)(((b.w[a] >> 41) << 1) | 1u) * 0x1.0p-24f;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float rad = sqrtf(-2.0f * logf(u[2 * p]));
    float sn, cs;
    sincospif(2.0f * u[2 * p + 1], &sn, &cs);
    z[2 * p] = rad * cs;
    z[2 * p + 1] = rad * sn;
  }
}

// Value of x held by the lane 32 positions away (lane l <-> l ^ 32), from
// one v_permlane32_swap.
__device__ __forceinline__ uint32_t swap_halves(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ uint64_t swap_halves64(uint64_t x) {
  return (uint64_t)swap_halves((uint32_t)x) |
         ((uint64_t)swap_halves((uint32_t)(x >> 32)) << 32);
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xFFFF0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Two floats -> packed bf16 pair (lo in bits 0..15), each rounded to nearest
// even (gfx950 lowers this to v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Split x into hi + lo with hi = bf16(x) and lo = bf16(x - hi); the residual
// x - hi is exact in fp32, so hi + lo carries about 16 significant bits.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  const __bf16 h = (__bf16)x;
  hi = __builtin_bit_cast(uint16_t, h);
  lo = f32_to_bf16(x - (float)h);
}

// Eight sign bits (bit e set = negative) -> eight bf16 +-1.0 values packed as
// an MFMA operand (element 2p in the low half of dword p).  With
// x = b | (b << 15), bit 2p of b sits at 2p and bit 2p+1 at 2p+16; shifting
// left by 15 - 2p moves them to bits 15 and 31, the two bf16 sign positions,
// and v_and_or_b32 keeps those and adds the +1.0 pattern.  x passes through an
// empty asm statement so the compiler no longer knows that b < 256 (with that
// knowledge it rewrites each shift as a quarter-rate multiply).  The two masks
// (k.m = 0x80008000, k.one = 0x3F803F80) come from sign_masks(), made opaque
// VGPR values once per kernel: one instruction may take only one scalar
// constant on this target, so with literal masks the compiler emitted a
// separate and and or per dword (r = 256 projection loop: 970 -> 842 VALU
// instructions per 64 MFMAs; wide-layer sketch 339 -> 318 us).
struct SignMasks {
  uint32_t m, one;
};
__device__ __forceinline__ SignMasks sign_masks() {
  SignMasks k{0x80008000u, 0x3F803F80u};
  asm volatile("" : "+v"(k.m), "+v"(k.one));
  return k;
}
__device__ __forceinline__ u32x4 signs_to_bf16x8(uint32_t byte, const SignMasks& k) {
  uint32_t x = byte | (byte << 15);
  asm("" : "+v"(x));
  u32x4 v;
  v[0] = ((x << 15) & k.m) | k.one;
  v[1] = ((x << 13) & k.m) | k.one;
  v[2] = ((x << 11) & k.m) | k.one;
  v[3] = ((x << 9) & k.m) | k.one;
  return v;
}

// Gaussian-basis entries of row i, columns 4q .. 4q+3: z * cr rounded to bf16
// (cr = 1/sqrt(r) as float).  Every kernel that needs Gaussian entries calls
// this one function, so they all see bit-identical values.
__device__ __forceinline__ void gaussian_entries_bf16(uint64_t seed,
                                                      uint64_t stream,
                                                      uint64_t q, uint64_t row,
                                                      float cr,
                                                      uint16_t out[4]) {
  float z[4];
  gaussian_block(seed, stream, q, row, z);
#pragma unroll
  for (int a = 0; a < 4; ++a) out[a] = f32_to_bf16(z[a] * cr);
}

// ---------------------------------------------------------------- MFMA
// gfx950 bf16 matrix cores, fp32 accumulation.
//   32x32x16: A row i = lane % 32, B column j = lane % 32; each lane supplies
//             8 K-values; D lane holds column lane % 32, rows
//             8 (v / 4) + 4 (lane / 32) + (v % 4) for v = 0..15.
//   16x16x32: A row i = lane % 16, B column j = lane % 16; each lane supplies
//             8 K-values; D lane holds column lane % 16, rows
//             4 (lane / 16) + v for v = 0..3.
// Which K index a (lane group, element) pair carries is irrelevant here:
// every caller feeds A and B with the same K assignment.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- loads
// Branch-free row loads.  Callers pass a column that lies inside the row's
// declared stride (ld >= round_up(ncols, 8) because ld % 8 == 0), so a whole
// aligned group can always be read; elements at or past `ncols` are then
// cleared with a bit mask (the padding may hold anything, including NaN).

// Mask keeping the first `valid` (0..8) bf16 of a 16-byte group, per dword.
__device__ __forceinline__ u32x4 keep_mask8(int valid) {
  u32x4 k;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int v = valid - 2 * p;
    k[p] = v >= 2 ? 0xFFFFFFFFu : v == 1 ? 0x0000FFFFu : 0u;
  }
  return k;
}

// 8 bf16 of `row` from element `col` (a multiple of 8); elements >= ncols
// read as zero.  Groups entirely past the end read the row's first group and
// are cleared.  Branch-free, so a run of these loads is issued back to back.
__device__ __forceinline__ u32x4 load_bf16x8_masked(const uint16_t* row, int col,
                                                    int ncols) {
  const int valid = ncols - col;
  const u32x4 v =
      *reinterpret_cast<const u32x4*>(row + (valid > 0 ? col : 0));
  return v & keep_mask8(valid);
}

// Interior fast path: the whole group is inside the row.
__device__ __forceinline__ u32x4 load_bf16x8(const uint16_t* row, int col) {
  return *reinterpret_cast<const u32x4*>(row + col);
}

// 2^x from the hardware instruction alone (v_exp_f32).  It equals exp2f
// wherever the result is a normal float; results below 2^-126 come out
// flushed instead of passing through exp2f's subnormal range fix (six more
// instructions per call).  Used for softmax weights 2^(a - max): a weight
// below 2^-126 of the row's largest is far under the fp32 resolution of the
// sums it joins.
__device__ __forceinline__ float exp2_normal(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- grid order
// Work-groups are dispatched round-robin over the 8 XCDs, so with a plain
// index -> tile map XCD x only ever gets tiles whose index is x mod 8.  On
// this part such tiles sit in the same slice of HBM address space (token
// blocks 256 KB apart, W column strips 512 B apart), and each XCD then streams
// from one slice while the others idle.  xcd_spread rotates the low three
// bits of `i` by `salt` inside every complete aligned group of 8 (a bijection
// on [0, n)), so each XCD's work-groups cover all residues.
__device__ __forceinline__ int xcd_spread(int i, int salt, int n) {
  return i < (n & ~7) ? ((i & ~7) | ((i + salt) & 7)) : i;
}

// Work-group L of a launch of n runs on XCD L mod 8.  xcd_runs gives it task
// (L mod 8) (n8 / 8) + L / 8, n8 = n rounded down to a multiple of 8 (the
// tail keeps its own index): each XCD takes one contiguous run of tasks.  With
// tasks numbered split-major (split s, d group g -> s groups + g) the
// work-groups of an XCD share one or two token splits, and their L2 fetches
// only those splits' P tiles instead of all of P.
__device__ __forceinline__ int xcd_runs(int L, int n) {
  const int n8 = n & ~7;
  return L < n8 ? (L & 7) * (n8 >> 3) + (L >> 3) : L;
}

// ---------------------------------------------------------------- LDS DMA
typedef __attribute__((address_space(3))) void lds_void;

// Byte address inside LDS of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// Direct global->LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes from `src` land at LDS byte address lds_base + 16 l.
// lds_base must be the same in every lane of the wave.  Written as inline
// assembly so that the compiler's wait-count pass, which does not see it,
// does not make every later LDS read wait for all outstanding vector loads;
// the caller orders its LDS reads after the copy with vm_wait<N>() and its
// LDS reads before a re-fill with lgkm_wait0().  M0 is saved and restored.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// The same copy with the non-temporal hint, for data read once (the layer
// input X of the projection).  Measured on the headline step with no input
// re-read from the Infinity Cache: temporal X copies made the step ~2 %
// slower (166.8 -> 170 us) and a lone call ~2 % slower.
__device__ __forceinline__ void lds_dma16_nt(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// Wait until at most N vector-memory instructions of this wave are in
// flight (they complete in issue order).
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lgkm_wait0() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

}  // namespace logra
