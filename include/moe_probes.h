/* Measurement probes (not part of the layer): what one MI355X reaches with
 * plain streams and back-to-back matrix-core instructions, so that a
 * benchmark can report its kernels against achieved as well as vendor peaks.
 * Same conventions as moe_mi355x.h: device pointers, 16-byte alignment,
 * work enqueued on `stream`, status codes of moe_status (0 = ok). */
#ifndef MOE_PROBES_H
#define MOE_PROBES_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` of `buf` once (each of 8192 workgroups of 256 threads
 * streams one contiguous chunk, 16 bytes per lane and load, eight loads in
 * flight per lane), keeping a running sum of the data that is
 * stored to sink[0] only in a case that does not occur for finite data, so
 * every byte is loaded and nothing is written.  bytes % 16 == 0, bytes > 0.
 * Errors: MOE_E_NULL, MOE_E_SHAPE, MOE_E_ALIGN, MOE_E_DEVICE. */
int moe_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t stream);

/* dst[i] = src[i] for `bytes` bytes (same chunks and loads as the read);
 * bytes % 16 == 0; the two ranges must not overlap.  Errors as
 * moe_probe_read, plus MOE_E_ALIAS. */
int moe_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

/* `iters` rounds of eight independent 32x32x16 bf16 MFMAs per wave in 1024
 * workgroups of four waves (32768 FLOP each: iters * 1024 * 4 * 8 * 32768
 * FLOP in all), register operands only; sink[0] is written only in a case
 * that does not occur.  1 <= iters <= 1<<20.  Errors: MOE_E_NULL,
 * MOE_E_SHAPE, MOE_E_DEVICE. */
int moe_probe_mfma(float* sink, int iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
