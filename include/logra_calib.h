/*
 * logra_calib.h - measurement helper shipped next to liblogra (in its own
 * library, liblogra_calib.so): a plain device copy whose achieved bandwidth
 * is the practical HBM ceiling the path's kernels are compared with.  It is
 * not part of the method.
 */
#ifndef LOGRA_CALIB_H
#define LOGRA_CALIB_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst <- src on stream s.  bytes % 16 == 0, both pointers 16-byte aligned
 * device memory, non-overlapping.  Returns 0, -1 (bad argument) or -3 (HIP
 * launch error). */
int logra_calib_copy(void* dst, const void* src, size_t bytes, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* LOGRA_CALIB_H */
