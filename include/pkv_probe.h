/*
 * pkv_probe.h -- C ABI of libpkv_probe, measurement kernels that give the
 * attention library's HBM figures a reference on the same GPU. Nothing on the
 * attention path calls them; the benchmark does, to report beside the
 * published 8 TB/s peak what a plain read-only stream reaches.
 *
 * pkv_probe_stream_read reads `bytes` bytes (a multiple of 16, buffer 16-byte
 * aligned) once, with 16-byte vector loads, and writes nothing unless the
 * XOR of everything read equals a fixed 32-bit value (then one word of
 * `sink`, a device int32, is written; with random data practically never).
 *   mode 0  plain: consecutive lanes read consecutive 16-byte chunks, and the
 *           grid strides over the buffer.
 *   mode 1  decode-shaped: the buffer is rows of row_bytes bytes (a multiple of
 *           256) holding row_bytes / 256 heads of 256 bytes; a wave reads one
 *           head's 256-byte slices of 64 consecutive rows at a time (16 lanes
 *           per slice, 16 loads in flight per lane), as the decode kernel
 *           reads one kv head's K or V.
 *   blocks  workgroups of 256 threads to launch (> 0).
 * Returns 0, or 1 for bad arguments, 3 when the launch fails. Asynchronous on
 * `stream` (a hipStream_t as void*).
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int pkv_probe_stream_read(const void *buf, size_t bytes, int32_t mode, int32_t row_bytes,
                          int32_t blocks, int32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
