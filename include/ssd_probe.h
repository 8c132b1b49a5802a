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

#include "ssd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Stream read_bytes from src and write_bytes to dst (both device memory, 16-byte aligned,
 * sizes multiples of 16, at most 2^31 16-byte items each) in one kernel on `stream`, the
 * reads and writes interleaved evenly in that ratio; the written values are unspecified.
 * sink: a device float that is written only in a case no finite input reaches.  Either
 * size may be 0 (write-only or read-only).  Errors: SSD_ERR_NULL_POINTER,
 * SSD_ERR_BAD_SHAPE, SSD_ERR_UNSUPPORTED (misaligned), SSD_ERR_HIP. */
ssd_status ssd_probe_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                            float* sink, ssd_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SSD_MI355X_PROBE_H */
