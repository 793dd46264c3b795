/*
 * qkv_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A plain, slow, scalar CPU statement of the DeepSeek-V4 style per-token
 * "q/kv prep" operator: RMSNorm of every 512-wide q head and of the kv row,
 * RoPE on the trailing 64 dims, q written back as bf16, the kv row's 448
 * leading dims quantized to FP8 E4M3 with one power-of-two (UE8M0) scale per
 * 64 elements, and the result inserted into a paged KV cache at slot_mapping.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no source with the GPU path and includes none
 * of its headers.  The product path never calls it.
 *
 * Pages this follows (cited by title and section):
 *   [FG] FlagGems-vllm PR 684, "fused_deepseek_v4_qnorm_rope_kv_rope_quant_insert
 *        backends, plus test and benchmark fixes".
 *   [SG] sglang PR 33358, "[Kernel] DSv4 flashmla norm-rope: K-tokens-per-block
 *        ILP to hide load latency".
 *   [MX] vLLM API page "vllm.models.minimax_m3.nvidia.ops.finalize_allreduce_norm"
 *        (the E4M3 / UE8M0 codec helpers it documents).
 *
 * Precision.  The pages compute this operator in fp32 between the bf16 input
 * and the bf16/FP8 outputs ([FG] "Ascend 910B" section: the fp32 upcast of q,
 * the fp32 norm output and the fp32 rope intermediate are held, and rounding
 * the normalized value to bf16 before the rotation is named as a mismatch with
 * the kernel's arithmetic).  Because the UE8M0 exponent is an integer decided by
 * floating point, the oracle takes every fp32 step in a fixed, stated order so
 * that a kernel following the same order reproduces it bit for bit.  Every
 * arithmetic operation below is a single IEEE-754 binary32 operation with
 * round-to-nearest-even (sqrtf, '/', '*', '+' and fmaf are all correctly
 * rounded); the file is compiled with -ffp-contract=off so that no product is
 * silently fused into an addition.
 *
 * Readings of points the pages leave open:
 *   R1 sum of squares: chunk l (l = 0..63) of 8 consecutive elements is summed
 *      left to right; the 64 chunk sums are then added pairwise, adjacent
 *      pairs first, in six levels.  [SG] Modifications says the reduction tree
 *      is part of the kernel's contract; [FG] Correctness shows that a changed
 *      lane assignment changes the variance bits.  The tree itself is not given.
 *   R2 inverse RMS: inv = 1 / sqrt(S/512 + eps), each of '/', '+', sqrt and the
 *      reciprocal correctly rounded; eps inside the root; the mean covers all
 *      512 dims, rope dims included ([SG] Motivation: RMSNorm over 512 dims).
 *   R3 weight: y = (x * inv) * w, two roundings; the q weight may be absent
 *      (weightless q norm, [FG] "Ascend 910B" baseline description).
 *   R4 RoPE: pairs are interleaved (448+2i, 449+2i); the rotated pair is
 *      (fma(a, c, -(b*s)), fma(a, s, b*c)) with the inner products rounded
 *      ([SG] Modifications item 4 pins the complex multiply to one fma form;
 *      [FG] "Ascend 910B" step list speaks of 2-D offsets for the RoPE pairs).
 *      The cos/sin table row holds cos_0..cos_31 then sin_0..sin_31 (fp32).
 *   R5 quantization input: the fp32 y (normalized and weighted, never rounded
 *      to bf16), blocks of 64 over dims 0..447 ([SG] Accuracy Tests: 7 groups of
 *      64 with UE8M0 exponents).  The scale exponent is the least e with
 *      amax <= 448 * 2^e, clamped to [-127, 127]; a zero block takes e = -127
 *      (scale byte 0).  This is the rounded-up exponent of [MX] _ue8m0_ceil,
 *      taken exactly rather than through amax * (1/448), and built from
 *      exponent bits rather than exp2 ([FG] "The seven test and benchmark
 *      fixes": the oracle's power-of-two scale is built exactly).
 *   R6 E4M3 (OCP e4m3fn): round to nearest, ties to even, subnormals kept,
 *      256 is a legal code, magnitudes above 448 saturate to 448 ([FG] "T-Head
 *      PPU-ZW810E" section; [MX] _f32x4_to_e4m3x4).  Signs are kept, so -0
 *      encodes as 0x80.
 *   R7 cache slot layout (not on the pages): a block of B slots holds B data
 *      records of 576 bytes (448 E4M3 codes, then 64 bf16 rope values,
 *      little-endian) followed by B scale records of 8 bytes (the 7 exponent
 *      bytes e+127, then a zero pad byte).  A slot outside [0, NB*B) writes
 *      nothing ([SG] Accuracy Tests: skipped slots stay untouched).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_HEAD_DIM 512
#define ORC_NOPE_DIM 448
#define ORC_ROPE_DIM 64
#define ORC_NPAIR 32
#define ORC_QBLOCK 64
#define ORC_NQBLOCK 7
#define ORC_SLOT_DATA 576
#define ORC_SLOT_SCALE 8
#define ORC_SLOT_BYTES 584

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

static float bits_to_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t float_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> fp32 is exact: the bf16 pattern is the upper half of the fp32 one. */
float orc_bf16_to_f32(uint16_t b) { return bits_to_float((uint32_t)b << 16); }

/* fp32 -> bf16, round to nearest, ties to even, by comparing the distances to
 * the two bf16 neighbours of |x| (computed exactly in double). */
uint16_t orc_f32_to_bf16(float x)
{
    uint32_t u = float_to_bits(x);
    if (isnan(x))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t sign = u & 0x80000000u;
    uint32_t mag = u & 0x7fffffffu;
    uint32_t lo = mag & 0xffff0000u;               /* largest bf16 magnitude <= |x| */
    if (lo == mag)
        return (uint16_t)((sign | lo) >> 16);
    uint32_t hi = lo + 0x10000u;                   /* smallest bf16 magnitude > |x| */
    double ax = (double)bits_to_float(mag);
    double dlo = (double)bits_to_float(lo);
    /* Past the largest finite bf16 the next step is 2^128 (IEEE overflow rule). */
    double dhi = (hi == 0x7f800000u) ? ldexp(1.0, 128) : (double)bits_to_float(hi);
    double below = ax - dlo, above = dhi - ax;
    uint32_t r;
    if (below < above)
        r = lo;
    else if (above < below)
        r = hi;
    else
        r = ((lo >> 16) & 1u) ? hi : lo;           /* tie: even bf16 mantissa */
    return (uint16_t)((sign | r) >> 16);
}

/* E4M3 (e4m3fn) code -> value.  Exponent bias 7, no infinities, S.1111.111 is NaN. */
double orc_e4m3_to_f64(uint8_t c)
{
    int neg = (c & 0x80) != 0;
    int e = (c >> 3) & 0xf;
    int m = c & 0x7;
    double v;
    if (e == 0xf && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                  /* subnormal: m * 2^-9 */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return neg ? -v : v;
}

/* fp32 -> E4M3, round to nearest, ties to even, saturating at 448 (R6).  The
 * value is split into a power of two and a significand in [1, 2); the
 * significand's fraction is rounded to 3 bits with nearbyint (ties-to-even
 * in the default rounding mode). */
uint8_t orc_f32_to_e4m3(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7f);
    double a = fabs((double)v);
    if (a < ldexp(1.0, -6)) {
        /* Subnormal range: the codes are m * 2^-9, m = 0..7; m = 8 is 2^-6,
         * whose code (exponent 1, mantissa 0) is also 8. */
        double m = nearbyint(a * 512.0);
        return (uint8_t)(sign | (uint8_t)m);
    }
    int E;
    double f = frexp(a, &E);                       /* a = f * 2^E, f in [0.5, 1) */
    int ex = E - 1;                                /* a = (2f) * 2^ex, 2f in [1, 2) */
    double q = nearbyint((2.0 * f - 1.0) * 8.0);   /* 3-bit fraction, 0..8 */
    if (q == 8.0) {
        q = 0.0;
        ex += 1;
    }
    int biased = ex + 7;
    if (biased > 15 || (biased == 15 && q == 7.0))
        return (uint8_t)(sign | 0x7e);             /* saturate to 448 */
    return (uint8_t)(sign | (biased << 3) | (int)q);
}

/* UE8M0 block exponent (R5): the least integer e with amax <= 448 * 2^e,
 * clamped to [-127, 127]; amax == 0 gives -127.  The comparisons are exact in
 * double (448 * 2^e is exact for every e used here). */
int orc_ue8m0_exponent(float amax)
{
    if (!(amax > 0.0f))
        return -127;
    double a = (double)amax;
    int e;
    frexp(a / 448.0, &e);                          /* first guess, may be off by one */
    while (a > ldexp(448.0, e))
        e += 1;
    while (a <= ldexp(448.0, e - 1))
        e -= 1;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

/* ------------------------------------------------------------------ */
/* One 512-wide row: RMSNorm, weight, RoPE                             */
/* ------------------------------------------------------------------ */

/* R1: sum of squares of 512 bf16 values in the fixed order. */
float orc_sum_squares(const uint16_t *x)
{
    float c[64];
    for (int l = 0; l < 64; ++l) {
        float acc = 0.0f;
        for (int k = 0; k < 8; ++k) {
            float v = orc_bf16_to_f32(x[8 * l + k]);
            acc = acc + v * v;                     /* v*v is exact for a bf16 v */
        }
        c[l] = acc;
    }
    for (int n = 64; n > 1; n /= 2)
        for (int i = 0; i < n / 2; ++i)
            c[i] = c[2 * i] + c[2 * i + 1];
    return c[0];
}

/* R2: inverse RMS from the sum of squares. */
float orc_inv_rms(float sum_sq, float eps)
{
    float mean_sq = sum_sq / 512.0f;
    float v = mean_sq + eps;
    float r = sqrtf(v);
    return 1.0f / r;
}

/* One row through norm, weight and rotation.
 *   x        512 bf16 inputs
 *   w        512 bf16 weights, or NULL for a weightless norm (R3)
 *   cs       64 fp32: cos_0..cos_31, sin_0..sin_31 of this token's position
 *   y        out: 512 fp32 normalized and weighted values, before the rotation
 *   z        out: 512 fp32 values after the rotation of dims 448..511
 *   stats    out (may be NULL): [0] = sum of squares, [1] = inverse RMS      */
void orc_row(const uint16_t *x, const uint16_t *w, float eps, const float *cs,
             float *y, float *z, float *stats)
{
    float s = orc_sum_squares(x);
    float inv = orc_inv_rms(s, eps);
    if (stats) {
        stats[0] = s;
        stats[1] = inv;
    }
    for (int j = 0; j < ORC_HEAD_DIM; ++j) {
        float t = orc_bf16_to_f32(x[j]) * inv;
        y[j] = w ? t * orc_bf16_to_f32(w[j]) : t;
        z[j] = y[j];
    }
    for (int i = 0; i < ORC_NPAIR; ++i) {          /* R4 */
        float a = y[ORC_NOPE_DIM + 2 * i];
        float b = y[ORC_NOPE_DIM + 2 * i + 1];
        float c = cs[i];
        float sn = cs[ORC_NPAIR + i];
        float bs = b * sn;
        float bc = b * c;
        z[ORC_NOPE_DIM + 2 * i] = fmaf(a, c, -bs);
        z[ORC_NOPE_DIM + 2 * i + 1] = fmaf(a, sn, bc);
    }
}

/* Quantize one block of 64 fp32 values (R5, R6).  Returns the scale byte. */
uint8_t orc_quant_block(const float *y, uint8_t *codes)
{
    float amax = 0.0f;
    for (int j = 0; j < ORC_QBLOCK; ++j)
        amax = fmaxf(amax, fabsf(y[j]));
    int e = orc_ue8m0_exponent(amax);
    float inv_scale = ldexpf(1.0f, -e);            /* exactly 2^-e */
    for (int j = 0; j < ORC_QBLOCK; ++j)
        codes[j] = orc_f32_to_e4m3(y[j] * inv_scale);
    return (uint8_t)(e + 127);
}

/* ------------------------------------------------------------------ */
/* Whole operator                                                      */
/* ------------------------------------------------------------------ */

/* Byte offsets of a slot's data and scale records inside the cache (R7).
 * Returns 0 and leaves the offsets alone when the slot writes nothing. */
int orc_slot_offsets(int64_t slot, int64_t num_blocks, int32_t block_size,
                     int64_t *data_off, int64_t *scale_off)
{
    if (slot < 0 || block_size <= 0 || slot >= num_blocks * (int64_t)block_size)
        return 0;
    int64_t blk = slot / block_size;
    int64_t s = slot % block_size;
    int64_t base = blk * (int64_t)block_size * ORC_SLOT_BYTES;
    *data_off = base + s * ORC_SLOT_DATA;
    *scale_off = base + (int64_t)block_size * ORC_SLOT_DATA + s * ORC_SLOT_SCALE;
    return 1;
}

/* Insert one token's kv row: codes of y[0..447] and bf16 of z[448..511]. */
static void insert_fp8_slot(const float *y, const float *z, uint8_t *cache,
                            int64_t data_off, int64_t scale_off)
{
    uint8_t *data = cache + data_off;
    uint8_t *scale = cache + scale_off;
    for (int b = 0; b < ORC_NQBLOCK; ++b)
        scale[b] = orc_quant_block(y + b * ORC_QBLOCK, data + b * ORC_QBLOCK);
    scale[ORC_NQBLOCK] = 0;
    for (int j = 0; j < ORC_ROPE_DIM; ++j) {
        uint16_t h = orc_f32_to_bf16(z[ORC_NOPE_DIM + j]);
        data[ORC_NOPE_DIM + 2 * j] = (uint8_t)(h & 0xff);
        data[ORC_NOPE_DIM + 2 * j + 1] = (uint8_t)(h >> 8);
    }
}

/* bf16-store variant of the insert: the slot holds the bf16 of all 512
 * values after the rotation (dims 0..447 are the normalized, weighted values;
 * 448..511 the rotated ones), 1024 bytes, no quantization ([SG] Motivation
 * and Speed Tests: the kernel's second store path).  Slot s of the cache is at
 * byte s * 1024, whatever the block split. */
static void insert_bf16_slot(const float *z, uint8_t *cache, int64_t slot)
{
    uint8_t *data = cache + slot * 1024;
    for (int j = 0; j < ORC_HEAD_DIM; ++j) {
        uint16_t h = orc_f32_to_bf16(z[j]);
        data[2 * j] = (uint8_t)(h & 0xff);
        data[2 * j + 1] = (uint8_t)(h >> 8);
    }
}

/* The operator over tokens [0, num_tokens).
 *   q_in, q_out   bf16 [T][H][512]; q_out may equal q_in (in place)
 *   kv            bf16 [T][512]
 *   q_w, kv_w     bf16 [512]; q_w may be NULL (weightless q norm)
 *   positions     int64 [T], each in [0, max_position)
 *   cos_sin       fp32 [max_position][64]
 *   slot_mapping  int64 [T]; outside [0, num_blocks*block_size) = skip
 *   cache         uint8 [num_blocks][block_size*584]
 *   nthreads      >= 1; tokens are independent, so they may run on several
 *                 threads (valid slots must be distinct, as for the kernel)
 * Returns 0, or -1 when an argument is unusable (nothing is written then). */
static int qkv_prep_store(int64_t num_tokens, int32_t num_heads,
                          const uint16_t *q_in, uint16_t *q_out, const uint16_t *kv,
                          const uint16_t *q_w, const uint16_t *kv_w,
                          const int64_t *positions, const float *cos_sin, int64_t max_position,
                          const int64_t *slot_mapping, uint8_t *cache, int64_t num_blocks,
                          int32_t block_size, float eps, int nthreads, int bf16_store)
{
    if (num_tokens < 0 || num_heads < 1 || max_position < 1 || nthreads < 1)
        return -1;
    for (int64_t t = 0; t < num_tokens; ++t)
        if (positions[t] < 0 || positions[t] >= max_position)
            return -1;

#pragma omp parallel for schedule(dynamic, 8) num_threads(nthreads)
    for (int64_t t = 0; t < num_tokens; ++t) {
        float y[ORC_HEAD_DIM], z[ORC_HEAD_DIM];
        const float *cs = cos_sin + positions[t] * 64;
        for (int32_t h = 0; h < num_heads; ++h) {
            int64_t row = (t * num_heads + h) * ORC_HEAD_DIM;
            orc_row(q_in + row, q_w, eps, cs, y, z, NULL);
            for (int j = 0; j < ORC_HEAD_DIM; ++j)
                q_out[row + j] = orc_f32_to_bf16(z[j]);
        }
        int64_t data_off, scale_off;
        if (orc_slot_offsets(slot_mapping[t], num_blocks, block_size, &data_off, &scale_off)) {
            orc_row(kv + t * ORC_HEAD_DIM, kv_w, eps, cs, y, z, NULL);
            if (bf16_store)
                insert_bf16_slot(z, cache, slot_mapping[t]);
            else
                insert_fp8_slot(y, z, cache, data_off, scale_off);
        }
    }
    return 0;
}

int orc_qkv_prep(int64_t num_tokens, int32_t num_heads,
                 const uint16_t *q_in, uint16_t *q_out, const uint16_t *kv,
                 const uint16_t *q_w, const uint16_t *kv_w,
                 const int64_t *positions, const float *cos_sin, int64_t max_position,
                 const int64_t *slot_mapping, uint8_t *cache, int64_t num_blocks,
                 int32_t block_size, float eps, int nthreads)
{
    return qkv_prep_store(num_tokens, num_heads, q_in, q_out, kv, q_w, kv_w, positions, cos_sin,
                          max_position, slot_mapping, cache, num_blocks, block_size, eps,
                          nthreads, 0);
}

/* Same operator with the bf16 cache: cache is uint8 [num_blocks][block_size*1024]. */
int orc_qkv_prep_bf16_store(int64_t num_tokens, int32_t num_heads,
                            const uint16_t *q_in, uint16_t *q_out, const uint16_t *kv,
                            const uint16_t *q_w, const uint16_t *kv_w,
                            const int64_t *positions, const float *cos_sin, int64_t max_position,
                            const int64_t *slot_mapping, uint8_t *cache, int64_t num_blocks,
                            int32_t block_size, float eps, int nthreads)
{
    return qkv_prep_store(num_tokens, num_heads, q_in, q_out, kv, q_w, kv_w, positions, cos_sin,
                          max_position, slot_mapping, cache, num_blocks, block_size, eps,
                          nthreads, 1);
}

/* ------------------------------------------------------------------ */
/* Cache reader                                                        */
/* ------------------------------------------------------------------ */

/* Dequantize-and-gather: the reader of this cache (the 1Cat-vLLM PR 1280 page,
 * change 5 "compressed KV gather", names dequantize_and_gather_k_cache as the
 * step that reads the FP8 DeepSeek-V4 cache back out; its layout is this
 * file's R7).  For each of n slots: dims 0..447 are
 * E4M3 code * 2^(byte - 127) of their 64-block, dims 448..511 the stored bf16
 * rope values; a slot outside [0, num_blocks*block_size) gives a row of
 * zeros.  The products are exact in fp32 (4 significant bits times a power of
 * two inside the fp32 range).  out: fp32 [n][512]. */
void orc_gather_dequant(const uint8_t *cache, int64_t num_blocks, int32_t block_size,
                        const int64_t *slots, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i) {
        float *row = out + i * ORC_HEAD_DIM;
        int64_t data_off, scale_off;
        if (!orc_slot_offsets(slots[i], num_blocks, block_size, &data_off, &scale_off)) {
            for (int j = 0; j < ORC_HEAD_DIM; ++j)
                row[j] = 0.0f;
            continue;
        }
        const uint8_t *data = cache + data_off;
        const uint8_t *scale = cache + scale_off;
        for (int j = 0; j < ORC_NOPE_DIM; ++j)
            row[j] = (float)ldexp(orc_e4m3_to_f64(data[j]), (int)scale[j / ORC_QBLOCK] - 127);
        for (int j = 0; j < ORC_ROPE_DIM; ++j)
            row[ORC_NOPE_DIM + j] = orc_bf16_to_f32(
                (uint16_t)(data[ORC_NOPE_DIM + 2 * j] | (data[ORC_NOPE_DIM + 2 * j + 1] << 8)));
    }
}

/* ------------------------------------------------------------------ */
/* Array helpers for the tests (elementwise, no arithmetic of their own) */
/* ------------------------------------------------------------------ */

void orc_f32_to_bf16_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_bf16(x[i]);
}

void orc_f32_to_e4m3_array(const float *x, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_e4m3(x[i]);
}

void orc_ue8m0_exponent_array(const float *amax, int32_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_ue8m0_exponent(amax[i]);
}

/* Per-row intermediates for a whole batch of rows (dumped by tests to settle
 * disputes bit for bit, [FG] "Ascend 910B": diff intermediates until the first
 * divergence).  x: [n][512], cs: [n][64]; y, z: [n][512]; stats: [n][2]. */
void orc_rows(int64_t n, const uint16_t *x, const uint16_t *w, float eps,
              const float *cs, float *y, float *z, float *stats)
{
    for (int64_t r = 0; r < n; ++r)
        orc_row(x + r * ORC_HEAD_DIM, w, eps, cs + r * 64, y + r * ORC_HEAD_DIM,
                z + r * ORC_HEAD_DIM, stats ? stats + 2 * r : NULL);
}

/* Quantize n rows of 448 fp32 values: codes [n][448], scale bytes [n][7]. */
void orc_quant_rows(int64_t n, const float *y, uint8_t *codes, uint8_t *scales)
{
    for (int64_t r = 0; r < n; ++r)
        for (int b = 0; b < ORC_NQBLOCK; ++b)
            scales[r * ORC_NQBLOCK + b] =
                orc_quant_block(y + r * ORC_NOPE_DIM + b * ORC_QBLOCK,
                                codes + r * ORC_NOPE_DIM + b * ORC_QBLOCK);
}

/* ------------------------------------------------------------------ */
/* MXFP8 norm-quant variant (a second workload for the same codec)     */
/* ------------------------------------------------------------------ */
/*
 * The residual-add + Gemma RMSNorm + MXFP8 quantization of the vLLM page
 * "vllm.models.minimax_m3.nvidia.ops.finalize_allreduce_norm" (class
 * _LamportGemmaRMSNormMxfp8Kernel and helpers _ue8m0_ceil, _ue8m0_inverse,
 * _f32x4_to_e4m3x4, _swizzled_scale_offset), without its all-reduce (one rank,
 * so the "sum of fragments" is the single input row).  Readings:
 *   M1 prenorm = bf16(x + residual), the sum in fp32 (the page adds the fp32
 *      fragments and the residual, then rounds to bf16); with no residual,
 *      prenorm = x.  residual_out, when given, receives prenorm.
 *   M2 sum of squares: chunks of 8 summed left to right, then adjacent pairs
 *      level by level; an odd element at the end of a level is carried up
 *      unchanged (the page's thread/warp/cluster order is not reproducible;
 *      this generalizes R1 to any multiple of 8).
 *   M3 inv = 1 / sqrt(S / hidden + eps), each step correctly rounded (the page
 *      uses an approximate rsqrt; this oracle takes the correctly rounded one).
 *   M4 normed = bf16((prenorm * inv) * (gamma + 1)), each product and the
 *      gamma + 1 rounded in fp32 (Gemma weight, the page's order).
 *   M5 per 32-element block: v = RN(amax * RN(1/448)); the scale byte is the
 *      biased exponent of v rounded up (the page's _ue8m0_ceil docstring),
 *      read as a definition: the least b >= 0 with v <= 2^(b - 127), at most
 *      254; 0 for v <= 0.  A power of two keeps its own exponent, anything
 *      else takes the next one up, and every v at or below 2^-127 gives 0.
 *      The inverse scale is 2^(127 - byte) (the page's _ue8m0_inverse
 *      docstring) while that power is a normal binary32 number, byte 1..253;
 *      byte 0 (a zero block) gives 0, and so does 254, whose power 2^-127
 *      lies below the normal range: the page's helper returns 0 there too.
 *   M6 code = E4M3 of RN(normed * inverse) clamped to +-448 first (satfinite).
 *   M7 codes row-major [m][hidden]; scale byte (row, col = block) at the
 *      128x4 swizzled offset col%4 + (col/4)*512 + (row%32)*16 +
 *      ((row%128)/32)*4 + (row/128)*128*padded_cols, padded_cols = cols rounded
 *      up to 4; the scale bytes of rows m .. (m rounded up to 128) - 1 are 0.
 */

static float f32_div(float a, float b) { return a / b; }

/* M2: sum of squares of n bf16 values (n a multiple of 8). */
float orc_sum_squares_n(const uint16_t *x, int64_t n)
{
    int64_t nc = n / 8;
    float *c = (float *)malloc(sizeof(float) * (size_t)(nc > 0 ? nc : 1));
    for (int64_t l = 0; l < nc; ++l) {
        float acc = 0.0f;
        for (int k = 0; k < 8; ++k) {
            float v = orc_bf16_to_f32(x[8 * l + k]);
            acc = acc + v * v;
        }
        c[l] = acc;
    }
    while (nc > 1) {
        int64_t half = nc / 2;
        for (int64_t i = 0; i < half; ++i)
            c[i] = c[2 * i] + c[2 * i + 1];
        if (nc % 2)
            c[half] = c[nc - 1];
        nc = half + nc % 2;
    }
    float s = nc ? c[0] : 0.0f;
    free(c);
    return s;
}

/* M5: the scale byte of v, from its defining inequality v <= 2^(b - 127),
 * compared exactly in double.  v is never NaN here (finite rows give a finite
 * amax); a NaN would read as "not positive". */
uint32_t orc_ue8m0_ceil_byte(float v)
{
    if (!(v > 0.0f))
        return 0;
    if (isinf(v))
        return 254;
    double a = (double)v;
    int b;
    frexp(a, &b);                                  /* 2^(b-1) <= a < 2^b */
    b += 127;                                      /* so a <= 2^(b - 127) holds */
    while (b > 0 && a <= ldexp(1.0, b - 1 - 127))  /* the least such b, not below 0 */
        b -= 1;
    if (b < 0)
        b = 0;
    return b > 254 ? 254u : (uint32_t)b;
}

/* M5: the inverse scale of a byte. */
float orc_ue8m0_inverse(uint32_t byte)
{
    if (byte == 0 || byte >= 254)
        return 0.0f;
    return (float)ldexp(1.0, 127 - (int)byte);
}

/* M7 */
int64_t orc_mxfp8_scale_offset(int64_t row, int64_t col, int64_t padded_cols)
{
    return col % 4 + (col / 4) * 512 + (row % 32) * 16 + ((row % 128) / 32) * 4 +
           (row / 128) * 128 * padded_cols;
}

/* Rows [0, m): x, residual (may be NULL), residual_out (may be NULL),
 * gamma: bf16; quant_out uint8 [m][hidden]; scale_out uint8
 * [round_up(m, 128)][padded_cols] in the swizzled order.  hidden must be a
 * positive multiple of 128.  Returns 0, or -1 for unusable arguments. */
int orc_mxfp8_norm_quant(int64_t m, int64_t hidden, const uint16_t *x, const uint16_t *residual,
                         uint16_t *residual_out, const uint16_t *gamma, float eps,
                         uint8_t *quant_out, uint8_t *scale_out)
{
    if (m < 0 || hidden <= 0 || hidden % 128)
        return -1;
    int64_t cols = hidden / 32;
    int64_t padded_cols = (cols + 3) / 4 * 4;
    int64_t rows_padded = (m + 127) / 128 * 128;
    uint16_t *pre = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)hidden);
    float *normed = (float *)malloc(sizeof(float) * (size_t)hidden);
    const float inv448 = f32_div(1.0f, 448.0f);
    for (int64_t r = 0; r < m; ++r) {
        const uint16_t *xr = x + r * hidden;
        for (int64_t j = 0; j < hidden; ++j) {
            if (residual) {
                float sum = orc_bf16_to_f32(xr[j]) + orc_bf16_to_f32(residual[r * hidden + j]);
                pre[j] = orc_f32_to_bf16(sum);
            } else {
                pre[j] = xr[j];
            }
            if (residual_out)
                residual_out[r * hidden + j] = pre[j];
        }
        float s = orc_sum_squares_n(pre, hidden);
        float mean_sq = f32_div(s, (float)hidden);
        float inv = 1.0f / sqrtf(mean_sq + eps);
        for (int64_t j = 0; j < hidden; ++j) {
            float g1 = orc_bf16_to_f32(gamma[j]) + 1.0f;
            float t = orc_bf16_to_f32(pre[j]) * inv;
            normed[j] = orc_bf16_to_f32(orc_f32_to_bf16(t * g1));
        }
        for (int64_t b = 0; b < cols; ++b) {
            float amax = 0.0f;
            for (int k = 0; k < 32; ++k)
                amax = fmaxf(amax, fabsf(normed[32 * b + k]));
            uint32_t byte = orc_ue8m0_ceil_byte(amax * inv448);
            float inverse = orc_ue8m0_inverse(byte);
            for (int k = 0; k < 32; ++k) {
                float v = normed[32 * b + k] * inverse;
                v = fminf(fmaxf(v, -448.0f), 448.0f);
                quant_out[r * hidden + 32 * b + k] = orc_f32_to_e4m3(v);
            }
            scale_out[orc_mxfp8_scale_offset(r, b, padded_cols)] = (uint8_t)byte;
        }
    }
    for (int64_t r = m; r < rows_padded; ++r)
        for (int64_t b = 0; b < padded_cols; ++b)
            scale_out[orc_mxfp8_scale_offset(r, b, padded_cols)] = 0;
    free(pre);
    free(normed);
    return 0;
}

/* The MXFP8 scale byte of n values (an array helper for the tests). */
void orc_ue8m0_ceil_byte_array(const float *v, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)orc_ue8m0_ceil_byte(v[i]);
}
