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
 *   mode 2  span: the buffer is cut into one contiguous span per wave, which
 *           the wave reads 1 KiB per load instruction with 16 loads in flight.
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

/* pkv_probe_issue times blocks of instructions as the prefill tile loop uses
 * them, to show what bounds that loop: one workgroup of 4 * waves_per_simd
 * waves per CU (its 96 KiB of LDS keeps a second workgroup off the CU), each
 * wave running 64 passes of one block and storing its shader-clock cycles in
 * cycles[block * 16 + wave] (device memory, blocks * 16 entries; entries of
 * absent waves are left as they are).
 *   mode 0  16 ds_read_b128 at the K-operand addresses (rows 256 B apart,
 *           XOR swizzle), then a wait
 *   mode 1  32 ds_read_b64_tr_b16 at the V^T-operand addresses, then a wait
 *   mode 2  16 v_mfma_f32_32x32x16_bf16 on 4 accumulators
 *   mode 3  32 independent v_exp_f32
 *   mode 4  32 v_fma_f32 on 32 chains
 *   mode 5  16 x (MFMA, one K-operand read); mode 6: 16 x (MFMA, two V^T
 *           reads); mode 7: 16 MFMAs with 24 reads, the tile's mix
 *   mode 8  waves 0-3 run 16 MFMAs while waves 4-7 (one beside each) run
 *           32 exp + 32 fma; mode 9: waves 0-3 alone; mode 10: waves 4-7
 *           alone (modes 8-10 need waves_per_simd 2)
 *   mode 11 16 x (MFMA, 4 independent v_fma_f32 of the same wave); mode 12:
 *           16 x (MFMA, 2 v_exp_f32 + 2 v_fma_f32); mode 13: 16 x (MFMA,
 *           8 v_fma_f32)
 *   mode 14 the tile mix of one wave: 16 MFMAs, 24 operand reads (as mode
 *           7) and 4 v_fma_f32 per MFMA; mode 15: the same with 2 v_exp_f32
 *           + 2 v_fma_f32 per MFMA; modes 16 and 17: modes 14 and 15 with
 *           the accumulators in AGPRs
 * waves_per_simd is 1, 2 or 4. Returns 0, 1 for bad arguments, 3 when the
 * launch fails. Asynchronous on `stream`. */
int pkv_probe_issue(int32_t mode, int32_t waves_per_simd, int32_t blocks, uint64_t *cycles,
                    int32_t *sink, void *stream);

/* pkv_probe_xcc launches n workgroups (n > 0) and has workgroup b write the
 * id of the XCD it runs on (the XCC_ID hardware register) to out[b] (device
 * memory, n int32). The prefill kernel's grid order assumes that the
 * hardware deals workgroups to the 8 XCDs round robin, so that workgroups
 * with equal b % 8 share an XCD (the first one's XCD depends on earlier
 * launches); this checks it. Returns 0, 1 for bad
 * arguments, 3 when the launch fails. Asynchronous on `stream`. */
int pkv_probe_xcc(int32_t *out, int32_t n, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
