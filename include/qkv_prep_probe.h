/*
 * qkv_prep_probe.h -- a measurement probe shipped in libqkv_prep.so next to
 * the operator: a plain streaming device-to-device copy.
 *
 * The pages measure the operator against a warm device-to-device copy of the
 * same card ("achievable bandwidth", FlagGems-vllm PR 684, section
 * "Performance against achievable bandwidth").  The runtime's own copy
 * (hipMemcpyAsync) is one such ceiling; this hand-written copy, built with
 * the same load/store idioms as the operator (16-byte non-temporal vector
 * accesses, several in flight per lane), is a second, usually stricter one.
 * It is not part of the operator.
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

#ifdef __cplusplus
}
#endif

#endif /* QKV_PREP_PROBE_H */
