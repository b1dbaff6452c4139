// Device copy and read used as the measured HBM ceilings next to the path's
// kernels (measurement helpers, not part of the method).  Copy: dst <- src, bytes a
// multiple of 16, both 16-byte aligned.  One work-group of 256 threads per
// 32 KB chunk; each thread issues its eight 16-byte non-temporal loads before
// its eight stores (loads branch-free: with a bounds test per load the
// compiler waited for each one before the next, 18.6 us instead of ~12.4 at
// 32 MiB).  Of the copy layouts measured on the MI355X (grid-stride
// loops, chunked work-groups, plain or non-temporal accesses, 512 to 65536
// work-groups) this one was the fastest at both 32 MiB and 1 GiB.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "logra_calib.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr size_t kChunk16 = (size_t)kThreads * kUnroll;   // 16-byte vectors per work-group

__global__ __launch_bounds__(kThreads) void copy_chunks(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, size_t n16) {
  const size_t b = (size_t)blockIdx.x * kChunk16 + threadIdx.x;
  // branch-free loads (past the end: the last vector again), so all eight
  // are in flight before the first store waits
  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const size_t i = b + (size_t)u * kThreads;
    v[u] = __builtin_nontemporal_load(src + (i < n16 ? i : n16 - 1));
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const size_t i = b + (size_t)u * kThreads;
    if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
  }
}

// Read-only stream: every 16-byte vector of src is loaded once (plain or
// non-temporal), eight per thread, 32 KB per work-group, folded with xor; the
// one store is taken only for an improbable fold value, so the loads stay
// live while nothing is written.
template <bool NT>
__global__ __launch_bounds__(kThreads) void read_chunks(const u32x4* __restrict__ src, size_t n16,
                                                        uint32_t* __restrict__ sink) {
  const size_t b = (size_t)blockIdx.x * kChunk16 + threadIdx.x;
  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const size_t i = b + (size_t)u * kThreads;
    const u32x4* p = src + (i < n16 ? i : n16 - 1);
    v[u] = NT ? __builtin_nontemporal_load(p) : *p;
  }
  u32x4 x = v[0];
#pragma unroll
  for (int u = 1; u < kUnroll; ++u) x ^= v[u];
  const uint32_t f = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (f == 0x9E3779B9u && threadIdx.x == 0) *sink = f;
}

}  // namespace

extern "C" int logra_calib_read(const void* src, size_t bytes, int nontemporal, void* sink,
                                hipStream_t s) {
  if (src == nullptr || sink == nullptr || bytes % 16 != 0) return -1;
  if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3)) return -1;
  if (bytes == 0) return 0;
  const size_t n16 = bytes / 16;
  const size_t blocks = (n16 + kChunk16 - 1) / kChunk16;
  if (blocks >= ((size_t)1 << 31)) return -1;
  if (nontemporal) {
    hipLaunchKernelGGL(read_chunks<true>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       static_cast<const u32x4*>(src), n16, static_cast<uint32_t*>(sink));
  } else {
    hipLaunchKernelGGL(read_chunks<false>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       static_cast<const u32x4*>(src), n16, static_cast<uint32_t*>(sink));
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int logra_calib_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (dst == nullptr || src == nullptr || bytes % 16 != 0) return -1;
  if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15) return -1;
  if (bytes == 0) return 0;
  const size_t n16 = bytes / 16;
  const size_t blocks = (n16 + kChunk16 - 1) / kChunk16;
  if (blocks >= ((size_t)1 << 31)) return -1;
  hipLaunchKernelGGL(copy_chunks, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
