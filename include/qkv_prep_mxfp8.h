/*
 * qkv_prep_mxfp8.h -- a second operator on the same codec, in the same
 * library: residual add + Gemma RMSNorm + MXFP8 (E4M3 values, one UE8M0 scale
 * per 32 elements) quantization of hidden-state rows, as the vLLM API page
 * "vllm.models.minimax_m3.nvidia.ops.finalize_allreduce_norm" describes for
 * _LamportGemmaRMSNormMxfp8Kernel and its helpers (_ue8m0_ceil,
 * _ue8m0_inverse, _f32x4_to_e4m3x4, _swizzled_scale_offset), without the
 * tensor-parallel all-reduce (one GPU: the row is this rank's input).
 *
 * Per row r (fp32 arithmetic, each step rounded to nearest even):
 *   p    = bf16(x + residual)  (or x when residual is NULL); written to
 *          residual_out when that is not NULL
 *   S    = sum of p_j^2: chunks of 8 left to right, then adjacent pairs level by
 *          level, an odd last element carried up unchanged
 *   inv  = 1 / sqrt(S / hidden + eps)   (correctly rounded; the page uses an
 *          approximate rsqrt)
 *   n_j  = bf16((p_j * inv) * (gamma_j + 1))
 *   per block of 32: v = RN(amax * RN(1/448)); byte = the biased exponent of v
 *          rounded up: the least b >= 0 with v <= 2^(b - 127), at most 254,
 *          and 0 for v <= 0 (so every v <= 2^-127 gives 0); inverse =
 *          2^(127 - byte) for bytes 1..253, 0 for byte 0 and for 254 (whose
 *          2^-127 is below the normal range); code_j =
 *          E4M3(clamp(RN(n_j * inverse), +-448)), round to nearest even
 *   codes: uint8 [m][hidden], row-major
 *   scales: the 128x4 swizzled layout, byte (row, col) at
 *          col%4 + (col/4)*512 + (row%32)*16 + ((row%128)/32)*4 + (row/128)*128*cols
 *          (cols = hidden/32), rows padded to a multiple of 128 with zero bytes.
 */
#ifndef QKV_PREP_MXFP8_H
#define QKV_PREP_MXFP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    const void *x;          /* bf16 [m][hidden]; 16-B aligned */
    const void *residual;   /* bf16 [m][hidden] or NULL; 16-B aligned */
    void *residual_out;     /* bf16 [m][hidden] or NULL; receives p; 16-B aligned */
    const void *gamma;      /* bf16 [hidden]; 16-B aligned */
    void *quant_out;        /* uint8 [m][hidden]; 16-B aligned */
    void *scale_out;        /* uint8 [qkv_prep_mxfp8_scale_bytes(m, hidden)]; 4-B aligned */
    int64_t m;              /* rows >= 0; 0 is a no-op */
    int32_t hidden;         /* a multiple of 128, at most 16384 */
    float eps;              /* >= 0, finite */
} qkv_prep_mxfp8_args;

/* Bytes of the swizzled scale buffer for m rows: round_up(m, 128) * hidden/32,
 * or -1 when m < 0, hidden is not a positive multiple of 128, or the size does
 * not fit in int64_t. */
int64_t qkv_prep_mxfp8_scale_bytes(int64_t m, int32_t hidden);

/* Enqueue on `stream` (a hipStream_t of HIP device `device`; NULL = that
 * device's null stream) and return.  The device is made current for the call
 * and the caller's current device is restored, as qkv_prep_run does with its
 * handle's device.  Return codes are those of qkv_prep.h:
 * QKV_PREP_ERR_INVALID_ARG (NULL pointer, negative m, bad eps),
 * QKV_PREP_ERR_MISALIGNED, QKV_PREP_ERR_UNSUPPORTED (hidden not a multiple of
 * 128 or above 16384, m > 2^31 - 128, or round_up(m, 128) * W >= 2^32: one
 * workgroup of W lanes per padded row, and the dispatch counts work-items in
 * 32 bits; W = 64 * ceil(hidden / 512) when that count K is odd and at most
 * 15, 32 * K when K is even, 32 * (K + 1) when K is odd and above 16),
 * QKV_PREP_ERR_NO_DEVICE (no such device), QKV_PREP_ERR_LAUNCH, and, with
 * QKV_PREP_SYNC=1 in the environment (the call then waits for the stream),
 * QKV_PREP_ERR_DEVICE for an asynchronous device error.
 * On an argument error nothing is launched.  No device memory is allocated
 * and only the one kernel is enqueued, so the call can be graph-captured. */
int qkv_prep_mxfp8_norm_quant(const qkv_prep_mxfp8_args *args, int device, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QKV_PREP_MXFP8_H */
