/*
 * qkv_prep_probe.h -- the measurement and verification probes, shipped in
 * their own library, libqkv_prep_probe.so, next to libqkv_prep.so.  None of
 * them is part of the operators; an application links libqkv_prep.so alone.
 *
 * Bandwidth ceilings.  The pages measure the operator against a warm
 * device-to-device copy of the same card (FlagGems-vllm PR 684, section
 * "Performance against achievable bandwidth").  The runtime's own copy
 * (hipMemcpyAsync) is one such ceiling; qkv_prep_probe_copy, written with the
 * same load/store idioms as the operator (16-byte non-temporal vector
 * accesses), is a second, usually stricter one; qkv_prep_probe_update is the
 * third: the operator rewrites q in place, and on MI355X in-place streaming
 * reaches a different rate from a copy between two buffers.
 *
 * Number-format probes.  qkv_prep_probe_convert and qkv_prep_probe_ue8m0 run
 * the operators' own device code for the E4M3, bf16 and UE8M0 rules on an
 * array, so a test can compare it with the oracle on every input pattern.
 *
 * All pointers are device pointers owned by the caller.  Return codes are
 * those of qkv_prep.h: 0 (QKV_PREP_OK), 1 (QKV_PREP_ERR_INVALID_ARG: NULL,
 * negative, out-of-range or misaligned argument; nothing is launched) and 5
 * (QKV_PREP_ERR_LAUNCH).  Each call enqueues one kernel on `stream` (a
 * hipStream_t; NULL = the null stream) of the current HIP device and returns.
 */
#ifndef QKV_PREP_PROBE_H
#define QKV_PREP_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copy `bytes` bytes from src to dst.  Both pointers 16-byte aligned, bytes a
 * multiple of 16, the ranges must not overlap.  bytes == 0 is a no-op.  The
 * same stream as qkv_prep_probe_stream(QKV_PREP_PROBE_COPY, NT, NT|SC1, 0, 64,
 * ...): the fastest copy of that probe's sweep. */
int qkv_prep_probe_copy(void *dst, const void *src, int64_t bytes, void *stream);

/* In-place streaming update of `bytes` bytes at buf: every 16-byte chunk is
 * read, its first 32-bit word (little-endian unsigned) is incremented by 1
 * with wrap-around, and the chunk is written back to the same address.  The
 * traffic is bytes read + bytes written.  buf 16-byte aligned, bytes a
 * multiple of 16; bytes == 0 is a no-op.  The same stream as
 * qkv_prep_probe_stream(QKV_PREP_PROBE_UPDATE, NT, NT|SC1, 0, 64, ...). */
int qkv_prep_probe_update(void *buf, int64_t bytes, void *stream);

/* Policy-selectable streams over `bytes` bytes (a multiple of 16), 16-byte
 * accesses, `lanes_per_block` lanes (64, 128, 256, 512 or 1024) per
 * workgroup and `depth` (1, 2, 4, 8 or 16) chunks per lane, lanes_per_block
 * chunks apart, whose loads are all issued before the lane's first store, for
 * comparing stream kinds, cache policies and shapes
 * on the device (the pages' own method of judging a kernel against what its
 * card can stream: FlagGems-vllm PR 684, "Performance against achievable
 * bandwidth").  kind:
 *   QKV_PREP_PROBE_READ (0)    reads src; dst is a 4-byte sink word (4-byte
 *                              aligned) that receives `key` only if some
 *                              chunk's four 32-bit words XOR to `key`;
 *   QKV_PREP_PROBE_WRITE (1)   writes dst: chunk i = {i mod 2^32, i >> 32,
 *                              key, ~key}; src must be NULL;
 *   QKV_PREP_PROBE_COPY (2)    copies src to dst (ranges must not overlap);
 *   QKV_PREP_PROBE_UPDATE (3)  in place at dst: the first 32-bit word of
 *                              every chunk is incremented with wrap-around;
 *                              src must be NULL.
 * load_policy / store_policy: the cache-policy bits of the loads / stores, a
 * combination of QKV_PREP_PROBE_SC0 (1), QKV_PREP_PROBE_NT (2) and
 * QKV_PREP_PROBE_SC1 (16).  Loads accept 0, NT or NT|SC1; stores accept 0,
 * NT, SC1, NT|SC1 or SC0|NT|SC1; the policy of an access the kind does not
 * make must be 0.  sleep = 1 (copy and update only) pauses each wavefront for
 * about 128 cycles between its loads' arrival and its stores; else 0.  With
 * depth > 1 the policies must be NT loads and NT|SC1 stores, and sleep 0.
 * xcd_order = 0 takes the workgroups' ranges in dispatch order (consecutive
 * workgroups, which the hardware deals round-robin over the 8 XCDs, take
 * consecutive ranges); xcd_order = 1 gives each XCD one contiguous eighth of
 * the buffer instead (the grid is padded to a multiple of 8 workgroups).
 * Written and read ranges 16-byte aligned.  Traffic: `bytes` for a read or a
 * write, 2 * bytes for a copy or an update.  bytes == 0 is a no-op after the
 * checks. */
enum { QKV_PREP_PROBE_READ = 0, QKV_PREP_PROBE_WRITE = 1, QKV_PREP_PROBE_COPY = 2, QKV_PREP_PROBE_UPDATE = 3 };
enum { QKV_PREP_PROBE_SC0 = 1, QKV_PREP_PROBE_NT = 2, QKV_PREP_PROBE_SC1 = 16 };
int qkv_prep_probe_stream(int32_t kind, int32_t load_policy, int32_t store_policy, int32_t sleep,
                          int32_t lanes_per_block, int32_t depth, int32_t xcd_order, void *dst, const void *src,
                          int64_t bytes, uint32_t key, void *stream);

/* The MXFP8 operator's memory access pattern with no arithmetic, for
 * measuring how close that operator runs to what its own loads and stores
 * allow: the same grid and workgroups (one per row, rows padded to 128), the
 * same non-temporal 16-byte loads and stores, per group of 64 chunks a
 * 16-byte gamma load before that group's 8-byte code stores and 4-byte
 * swizzled scale words, and zero words for the padding rows.  x, residual and
 * residual_out are [m][hidden] 16-bit elements and gamma [hidden] 16-bit
 * elements (16-byte aligned), codes [m][hidden] bytes (8-byte aligned),
 * scales the 128x4 swizzled layout of qkv_prep_mxfp8.h (4-byte aligned,
 * qkv_prep_mxfp8_scale_bytes(m, hidden) bytes).  hidden a multiple of 512
 * from 512 to 16384 whose group count hidden / 512 is even or at most 15.
 * With w the four 32-bit words of a 16-byte chunk of x (of x XOR residual
 * with bit 0) and y those of the same chunk of gamma, streams:
 *   bit 0 (1)  reads residual, writes residual_out = x XOR residual;
 *   bit 1 (2)  writes the codes, chunk c's 8 bytes = {w0^w1^y0^e, w2^w3^y1};
 *   bit 2 (4)  writes the scale word of every 4 chunks (columns 4j..4j+3 of
 *              the row) = w0^w3^y3^e of its first chunk, and zero words in
 *              the padding rows;
 *   bit 3 (8)  adds the operator's LDS barrier, after which e = word 0 of
 *              the row's first chunk (e = 0 without it).
 * At least one of bits 0-2; gamma may be NULL without bits 1-2, residual and
 * residual_out without bit 0.  m == 0 is a no-op after the checks. */
int qkv_prep_probe_mxfp8_pattern(const void *x, const void *residual, const void *gamma, void *residual_out,
                                 void *codes, void *scales, int64_t m, int32_t hidden, int32_t streams,
                                 void *stream);

/* The operator's fp32 conversions on n values of `in`:
 * e4m3_out[i] = the E4M3 code of in[i] (OCP e4m3fn, round to nearest even;
 * defined for |in[i]| <= 448, the range the operator converts) and
 * bf16_out[i] = the bf16 of in[i] (round to nearest even; defined for finite
 * values).  convert selects the path as in qkv_prep_config: 1 = integer
 * rounding, 2 = the gfx950 conversion instructions.  Either output may be
 * NULL.  in 16-byte aligned, e4m3_out 4-byte aligned, bf16_out 8-byte
 * aligned, n >= 0 a multiple of 4 and below 2^33. */
int qkv_prep_probe_convert(const float *in, int64_t n, void *e4m3_out, void *bf16_out, int32_t convert,
                           void *stream);

/* The two UE8M0 rules on n values of `in` (fp32, 4-byte aligned, n < 2^38):
 *   op_byte_out[i]  (uint8) the main operator's scale byte e + 127 of a block
 *                   whose amax is in[i]: e is the least integer with
 *                   amax <= 448 * 2^e, clamped to [-127, 127] (defined for
 *                   finite in[i] >= 0);
 *   mx_byte_out[i]  (uint8) the MXFP8 operator's scale byte of v = in[i]: the
 *                   least b >= 0 with v <= 2^(b - 127), at most 254, and 0
 *                   for v <= 0 (defined for finite v);
 *   mx_inverse_out  (fp32 [256], 4-byte aligned) the MXFP8 inverse scale of
 *                   every byte 0..255: 2^(127 - byte) for 1..253, else 0.
 * Any output may be NULL; with n == 0 only mx_inverse_out is written. */
int qkv_prep_probe_ue8m0(const float *in, int64_t n, void *op_byte_out, void *mx_byte_out,
                         void *mx_inverse_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QKV_PREP_PROBE_H */
