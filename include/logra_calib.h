/*
 * logra_calib.h - measurement helper shipped next to liblogra (in its own
 * library, liblogra_calib.so): a plain device copy and a plain device read
 * whose achieved bandwidths are the practical HBM ceilings the path's
 * kernels are compared with.  They are not part of the method.
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

/* Reads every byte of src once on stream s (plain loads, or non-temporal
 * ones with nontemporal != 0) and writes nothing, except possibly 4 bytes at
 * sink: the practical ceiling of a read-only stream such as the sketch's
 * two passes over X and dY.  bytes % 16 == 0, src 16-byte and sink 4-byte
 * aligned device memory.  Returns 0, -1 (bad argument) or -3 (HIP launch
 * error). */
int logra_calib_read(const void* src, size_t bytes, int nontemporal, void* sink, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* LOGRA_CALIB_H */
