/*
 * conv2d_probe.h -- measurement aid exported by libconv2d.so.
 *
 * The scope's measurement asks for the HBM-bound kernels (depthwise, the
 * fused pointwise/depthwise pairs) to be reported against the attainable
 * HBM bandwidth on one GPU, not only against the 8 TB/s peak.
 * conv2d_probe_copy is that reference: a plain streaming copy written the way
 * those kernels move data (16-byte vector loads and stores, every load of a
 * thread issued before its stores), timed by the benchmark at the byte count
 * of each kernel it is compared with.
 */
#ifndef CONV2D_PROBE_MI355X_H
#define CONV2D_PROBE_MI355X_H

#include <stdint.h>

#include "conv2d.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copy `bytes` bytes from device pointer src to device pointer dst on
 * `stream` (hipStream_t, null = default stream), asynchronously.  Both
 * pointers must be 16-byte aligned and bytes a multiple of 16; the ranges
 * must not overlap.  Errors: INVALID_ARG for null or misaligned pointers or
 * a byte count that is not a multiple of 16; ALIAS for overlapping ranges;
 * HIP if the launch fails.  The library allocates nothing. */
CONV2D_API conv_status_t conv2d_probe_copy(void* dst, const void* src, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONV2D_PROBE_MI355X_H */
