/*
 * axr_probe.h -- bandwidth probes shipped with libaxr for measurement.
 *
 * Not part of the method: plain streaming kernels that report the HBM rate a
 * bare stream (and the LDS rate a bare table-read loop) reaches on the
 * running machine, so that the scoring and quantization kernels can be
 * quoted against it as well as against the published peak.  All calls
 * validate their arguments before any HIP call,
 * enqueue one kernel on `stream` (a hipStream_t cast to void*, NULL = default
 * stream), never synchronise and allocate nothing.  Return 0 on success, -1 on
 * a bad argument, -4 when the launch fails.
 */
#ifndef AXR_PROBE_H
#define AXR_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of device memory at `buf` (16-byte aligned, bytes a
 * multiple of 16) with 16-byte loads.  `sink` is a device uint32 that the
 * kernel writes only in a case that cannot occur for real data; it keeps the
 * loads from being optimised away. */
int axr_probe_read_stream(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* Reads `in_bytes` bytes at `in` (16-byte aligned, multiple of 16) and writes
 * `out_bytes` bytes at `out` (4-byte aligned, multiple of 4); every block
 * reads a contiguous share of the input and then writes a contiguous share of
 * the output. */
int axr_probe_read_write(const void* in, int64_t in_bytes, void* out, int64_t out_bytes,
                         void* stream);

/* LDS read rate: 256 blocks of 1024 threads (one per CU), each reading its
 * own 128 KiB LDS array with 16-byte reads, iters x 16 reads per thread, in
 * the score kernel's table pattern: the 16 lanes of each quarter-wave read 16
 * distinct 16-byte columns of 256-byte rows chosen by a per-lane hash.  Bytes
 * read per CU: 1024 * 16 * iters * 16.  `out` is a device uint32 [262144]
 * (one checksum per thread, 4-byte aligned); iters in [1, 65536]. */
int axr_probe_lds_read(int iters, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AXR_PROBE_H */
