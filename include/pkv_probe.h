/* pkv_probe.h -- a measurement probe beside the attention library (libpkvprobe.so), not part of the path.
 *
 * pkv_probe_stream_read: the simplest kernel that moves a decode launch's bytes in the decode kernel's work
 * decomposition.  Workgroup g of `groups` (512 threads each, one per tile, in the order the decode launch
 * dispatches its tiles) reads its own contiguous run of 16-byte chunks x[off16[g] .. off16[g] + len16[g]) (clamped
 * into the x_bytes of x)
 * (non-temporal loads, eight in flight per thread) and then writes write_bytes of y at y + g * write_bytes.
 * bench.py --floor times it on a workload's exact tile sizes: what the plainest kernel with one workgroup per tile
 * takes, a reference for the decode launch (not a bound: pipelined waves can keep more bytes in flight).
 *   x: device, 16-byte aligned, x_bytes long; off16: device, [groups] int64 chunk offsets; len16: device,
 *   [groups] int32 chunk counts (negative reads as 0); y: device, 16-byte aligned, groups * write_bytes bytes (may be
 *   null when write_bytes is 0);
 *   write_bytes: a multiple of 16, >= 0.  stream: a hipStream_t (null: the default stream).  The caller owns every
 *   buffer.  Returns 0 on success, 1 on invalid arguments (nothing launched), 2 when the launch failed.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* built with hidden visibility; the entry point is exported */
__attribute__((visibility("default"))) int pkv_probe_stream_read(const void *x, int64_t x_bytes,
                                                                 const int64_t *off16, const int32_t *len16, void *y,
                                                                 int32_t groups, int32_t write_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif
