/*
 * qkv_prep_probe.h -- probes shipped in libqkv_prep.so next to the operator:
 * a plain streaming device-to-device copy and a streaming in-place update
 * (read and write the same bytes, as the operator does with q), used as
 * bandwidth ceilings; and the operator's fp32 -> E4M3 / bf16 conversions on
 * an array, for exhaustive checks of the conversion instructions.
 *
 * The pages measure the operator against a warm device-to-device copy of the
 * same card ("achievable bandwidth", FlagGems-vllm PR 684, section
 * "Performance against achievable bandwidth").  The runtime's own copy
 * (hipMemcpyAsync) is one such ceiling; this hand-written copy, built with
 * the same load/store idioms as the operator (16-byte non-temporal vector
 * accesses), is a second, usually stricter one.  The in-place update is the
 * third: the operator rewrites q in place, and on MI355X in-place streaming
 * reaches a different rate from a copy between two buffers.  None of them is
 * part of the operator.
 */
#ifndef QKV_PREP_PROBE_H
#define QKV_PREP_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copy `bytes` bytes from device pointer src to device pointer dst on
 * `stream` (a hipStream_t; NULL = null stream) and return.  Both pointers
 * 16-byte aligned, bytes a multiple of 16, the ranges must not overlap.
 * Returns 0 (QKV_PREP_OK), 1 (invalid argument: NULL, negative or unaligned),
 * or 5 (launch failed).  bytes == 0 is a no-op. */
int qkv_prep_probe_copy(void *dst, const void *src, int64_t bytes, void *stream);

/* In-place streaming update of `bytes` bytes at device pointer buf on
 * `stream`: every 16-byte chunk is read, its first 32-bit word (little-endian
 * unsigned) is incremented by 1 with wrap-around, and the chunk is written
 * back to the same address.  The traffic is bytes read + bytes written.
 * buf 16-byte aligned, bytes a multiple of 16.  Returns 0, 1 (invalid
 * argument: NULL, negative or unaligned) or 5 (launch failed); bytes == 0 is a
 * no-op. */
int qkv_prep_probe_update(void *buf, int64_t bytes, void *stream);

/* Run the operator's own fp32 conversions on n values of `in`, on `stream`:
 * e4m3_out[i] = the E4M3 code of in[i] (OCP e4m3fn, round to nearest even;
 * defined for |in[i]| <= 448, the range the operator converts) and
 * bf16_out[i] = the bf16 of in[i] (round to nearest even; defined for finite
 * values).  convert selects the path as in qkv_prep_config: 1 = integer
 * rounding, 2 = the gfx950 conversion instructions.  Either output may be
 * NULL.  in 16-byte aligned, e4m3_out 4-byte aligned, bf16_out 8-byte
 * aligned, n >= 0 a multiple of 4 and below 2^33.  Returns 0, 1 (invalid or
 * misaligned argument) or 5 (launch failed).  A verification probe: it lets a
 * test compare the device conversions with a reference on every input
 * pattern. */
int qkv_prep_probe_convert(const float *in, int64_t n, void *e4m3_out, void *bf16_out, int32_t convert,
                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QKV_PREP_PROBE_H */
