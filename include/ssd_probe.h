/*
 * ssd_probe.h -- measurement aid shipped with the SSD library (not a step of the scan).
 *
 * The benchmark states each HBM-bound kernel's achieved bandwidth against the spec peak and
 * against what this device sustains for the same mix of read and written bytes; this call
 * measures the latter with a plain streaming kernel.
 */
#ifndef SSD_MI355X_PROBE_H
#define SSD_MI355X_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "ssd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Stream read_bytes from src and write_bytes to dst (both device memory, 16-byte aligned,
 * sizes multiples of 16, at most 2^31 16-byte items each) in one kernel on `stream`, the
 * reads and writes interleaved evenly in that ratio; the written values are unspecified.
 * sink: a device float that is written only in a case no finite input reaches.  Either
 * size may be 0 (write-only or read-only).
 * variant (0 .. 11) picks the access form, since the fastest one depends on the mix:
 * bit 0 set = plain stores (else non-temporal), bit 1 set = each role's workgroups stride
 * through its buffer together (else each takes one contiguous share), variant >> 2 =
 * 0, 1, 2 for a grid of 2048, 4096 or 8192 workgroups.  Errors: SSD_ERR_NULL_POINTER,
 * SSD_ERR_BAD_SHAPE (sizes, variant), SSD_ERR_UNSUPPORTED (misaligned), SSD_ERR_HIP. */
ssd_status ssd_probe_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                            float* sink, int32_t variant, ssd_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SSD_MI355X_PROBE_H */
