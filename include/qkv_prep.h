/*
 * qkv_prep.h -- C ABI of the fused DeepSeek-V4 style q/kv prep operator for
 * AMD Instinct MI355X (gfx950).
 *
 * One call does, for every token t of a batch:
 *   - RMSNorm of each of the H q heads (512 dims), RoPE on the head's trailing
 *     64 dims, and the result written back into q as bf16, in place;
 *   - RMSNorm of the kv row (512 dims) and RoPE on its trailing 64 dims;
 *   - FP8 E4M3 quantization of the kv row's leading 448 dims with one
 *     power-of-two (UE8M0) scale per 64 elements;
 *   - insertion of the codes, the 64 rotated rope values (bf16) and the 7
 *     scale bytes into a paged KV cache at slot_mapping[t].
 *
 * The operation is the one named fused_deepseek_v4_qnorm_rope_kv_rope_quant_insert
 * on the FlagGems-vllm PR 684 page ("...backends, plus test and benchmark fixes",
 * sections "What the token tiling does" and "T-Head PPU-ZW810E"), whose kv half
 * is the norm-rope-store kernel of the sglang PR 33358 page ("DSv4 flashmla
 * norm-rope: K-tokens-per-block ILP", Motivation and Accuracy Tests).  The
 * exact arithmetic (reduction order, rounding of every fp32 step, E4M3 and
 * UE8M0 rules) is stated below under "Numerics".
 *
 * All tensor pointers are device pointers owned by the caller.  Nothing here
 * allocates device memory, and no PyTorch or HIP type appears in the
 * signatures (the stream is passed as void*, a hipStream_t).
 */
#ifndef QKV_PREP_H
#define QKV_PREP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKV_PREP_HEAD_DIM 512
#define QKV_PREP_NOPE_DIM 448
#define QKV_PREP_ROPE_DIM 64
#define QKV_PREP_QUANT_BLOCK 64
#define QKV_PREP_NUM_SCALES 7
/* Bytes of one cache slot: 576 data bytes + 8 scale bytes. */
#define QKV_PREP_SLOT_DATA_BYTES 576
#define QKV_PREP_SLOT_SCALE_BYTES 8
#define QKV_PREP_SLOT_BYTES 584

/* Return codes.  On any code other than QKV_PREP_OK from an argument check,
 * nothing was launched and no output was touched.  The launch itself is
 * checked with hipGetLastError right after it, so a refused launch is reported
 * by the call that made it; an error of the running kernel is asynchronous,
 * and QKV_PREP_SYNC=1 in the environment makes every call wait for its stream
 * and report such an error as QKV_PREP_ERR_DEVICE.  The FlagGems-vllm PR 684
 * page ("The seven test and benchmark fixes") describes a backend where a failed
 * launch surfaced only at the next launch, several frames from its cause: these
 * two checks keep the error with the call that caused it. */
enum {
    QKV_PREP_OK = 0,
    QKV_PREP_ERR_INVALID_ARG = 1,   /* NULL pointer, negative size, bad field */
    QKV_PREP_ERR_UNSUPPORTED = 2,   /* shape outside what the kernel implements */
    QKV_PREP_ERR_MISALIGNED = 3,    /* a pointer breaks the alignment rule below */
    QKV_PREP_ERR_NO_DEVICE = 4,     /* no HIP device, or the device index is out of range */
    QKV_PREP_ERR_LAUNCH = 5,        /* the runtime refused the launch (hipGetLastError) */
    QKV_PREP_ERR_DEVICE = 6         /* an asynchronous device error, seen in sync mode */
};

typedef struct qkv_prep *qkv_prep_t;

/* Fixed per-handle configuration. */
typedef struct {
    int32_t num_heads;        /* H >= 1 q heads per token */
    int32_t head_dim;         /* must be 512 */
    int32_t rope_dim;         /* must be 64 (the trailing dims of each row) */
    int32_t block_size;       /* B >= 1 cache slots per block */
    float eps;                /* >= 0, finite; added to the mean square */
    int32_t rows_per_wave;    /* 0 = launch heuristic; 1 = one q row per wavefront;
                                 2 or 4 = that many consecutive heads of one
                                 token per wavefront, one after another (the
                                 heuristic's choice is described at
                                 qkv_prep_launch_shape) */
    int32_t waves_per_block;  /* 0 = launch heuristic; 1, 2, 4 or 8 forces it (the
                                 heuristic takes 2 with two heads per wavefront
                                 where it takes several kv tokens per kv
                                 wavefront; else 1) */
    int32_t convert;          /* 0 = heuristic, 1 = integer bf16/E4M3 rounding,
                                 2 = gfx950 conversion instructions; both give
                                 the same bits (tests check this) */
    int32_t kv_store;         /* QKV_PREP_KV_FP8 (0): the FP8 + UE8M0 slot below;
                                 QKV_PREP_KV_BF16 (1): the bf16-store path of the
                                 sglang PR 33358 page (Motivation: the kernel's
                                 second store path), a slot of 1024 bytes holding
                                 the bf16 of all 512 values after the rotation
                                 (dims 0..447 normalized and weighted, 448..511
                                 rotated); slot s at byte s * 1024 */
    int32_t kv_per_wave;      /* 0 = launch heuristic; 1, 2 or 4 = that many
                                 consecutive tokens' kv rows per wavefront, all
                                 their loads issued together (the heuristic's
                                 choice is described at qkv_prep_launch_shape) */
} qkv_prep_config;

#define QKV_PREP_KV_FP8 0
#define QKV_PREP_KV_BF16 1
#define QKV_PREP_BF16_SLOT_BYTES 1024

/* Per-call tensors.  Layouts are dense row-major.  (kv_cache below is the
 * FP8 layout; with kv_store = QKV_PREP_KV_BF16 it is uint8
 * [num_blocks][B * 1024] instead.)
 *   q            bf16 [T][H][512], read and overwritten in place; 16-B aligned
 *   kv           bf16 [T][512], read only; 16-B aligned
 *   q_norm_w     bf16 [512], or NULL for a weightless q RMSNorm; 16-B aligned
 *   kv_norm_w    bf16 [512]; 16-B aligned
 *   positions    int64 [T]; each in [0, max_position) (precondition)
 *   cos_sin      fp32 [max_position][64]: cos_0..cos_31 then sin_0..sin_31 of
 *                the token's angles; 16-B aligned
 *   slot_mapping int64 [T]; a value outside [0, num_blocks * B) skips that
 *                token's cache write; valid values must be distinct
 *   kv_cache     uint8 [num_blocks][B * 584]; 16-B aligned.  Block b holds B
 *                data records of 576 B (448 E4M3 codes, then 64 bf16 rope values)
 *                followed by B scale records of 8 B (7 exponent bytes e + 127,
 *                then a zero pad byte).  Slot s of block b: data at
 *                b*B*584 + s*576, scales at b*B*584 + B*576 + s*8.          */
typedef struct {
    void *q;
    const void *kv;
    const void *q_norm_w;
    const void *kv_norm_w;
    const int64_t *positions;
    const float *cos_sin;
    int64_t max_position;     /* >= 1 rows in cos_sin */
    const int64_t *slot_mapping;
    void *kv_cache;
    int64_t num_blocks;       /* >= 0 */
    int64_t num_tokens;       /* T >= 0; T == 0 is a no-op */
} qkv_prep_args;

/* What qkv_prep_run launches for a given T (for logging and sweeps). */
typedef struct {
    int32_t rows_per_wave;
    int32_t waves_per_block;
    int32_t convert;          /* 1 integer, 2 instructions */
    int32_t kv_per_wave;      /* tokens' kv rows per kv wavefront (1, 2 or 4) */
    int64_t kv_blocks;        /* workgroups that handle kv rows */
    int64_t q_blocks;         /* workgroups that handle q rows */
    int64_t grid;             /* kv_blocks + q_blocks; a grid of more than
                                 (2^32 - 1) / (64 * waves_per_block) workgroups
                                 (a dispatch counts work-items in 32 bits) is
                                 enqueued as consecutive dispatches of that
                                 many workgroups, in order */
    int64_t kv_period;        /* 0: the kv workgroups come first in the grid;
                                 else (two heads and four kv tokens per
                                 wavefront, from 2^18 q rows) kv workgroup j
                                 is grid index j * kv_period, an odd spacing
                                 >= 3 that spreads them over the first 55-75%
                                 of the grid */
} qkv_prep_launch;

/* Arguments of the cache reader (qkv_prep_gather).
 *   kv_cache   uint8 [num_blocks][B * 584], an FP8 + UE8M0 cache written by
 *              qkv_prep_run (layout above); 16-B aligned
 *   slots      int64 [n]: the slots to read; one outside [0, num_blocks * B)
 *              reads as a row of zeros
 *   out        [n][512] of out_dtype; 16-B aligned
 *   out_dtype  QKV_PREP_OUT_F32 (0) or QKV_PREP_OUT_BF16 (1)              */
typedef struct {
    const void *kv_cache;
    int64_t num_blocks;
    const int64_t *slots;
    int64_t n;                /* >= 0; 0 is a no-op */
    void *out;
    int32_t out_dtype;
} qkv_prep_gather_args;

#define QKV_PREP_OUT_F32 0
#define QKV_PREP_OUT_BF16 1

/* Create a handle for device `device`.  Validates cfg, reads the device's
 * compute-unit count for the launch heuristic, and stores host state only.
 * Returns QKV_PREP_ERR_NO_DEVICE when no HIP device exists or the index is
 * out of range, QKV_PREP_ERR_INVALID_ARG / _UNSUPPORTED for a bad cfg (and
 * QKV_PREP_ERR_INVALID_ARG if the small host allocation fails).
 * *out is set only on success; release it with qkv_prep_destroy. */
int qkv_prep_create(const qkv_prep_config *cfg, int device, qkv_prep_t *out);

/* Enqueue the operator on `stream` (a hipStream_t; NULL = the null stream)
 * of the handle's device and return.  The arguments are checked on the host
 * first (pointers, sizes, 16-B alignment); nothing is launched on error.
 * Preconditions not checked on the device: positions in range (an
 * out-of-range position is clamped into the table, so memory stays in bounds,
 * but that token's output is unspecified), distinct valid slots, finite
 * inputs.  With QKV_PREP_SYNC=1 in the environment the call also waits for
 * the stream and reports a device error as QKV_PREP_ERR_DEVICE.  With
 * QKV_PREP_LOG=1 the handle prints its launch shape to stderr whenever it
 * differs from the last one it printed (once per shape in a steady run).
 * Both variables are read by qkv_prep_create.
 * The handle's configuration is read only here (the log's last-shape record
 * is atomic), so concurrent calls on different streams are safe.  The call
 * allocates no device memory and enqueues nothing but the kernel (no memset,
 * no copy; one dispatch, or consecutive dispatches of the same kernel for a
 * grid past 2^32 work-items, from about 2^26 q rows), so it can be captured
 * in a HIP graph.
 *
 * Numerics (all fp32, each step rounded to nearest even):
 *   S     = sum of x_j^2: chunk l (8 consecutive dims) summed left to right,
 *           then the 64 chunk sums added pairwise, adjacent pairs first;
 *   inv   = 1 / sqrt(S/512 + eps)   (division and sqrt correctly rounded);
 *   y_j   = (x_j * inv) * w_j       (or x_j * inv with no q weight);
 *   RoPE  on pairs (448+2i, 449+2i) with c = cos_i, s = sin_i:
 *           a' = fma(a, c, -(b*s)),  b' = fma(a, s, b*c);
 *   q out = bf16(round to nearest even) of y (dims 0..447) and the rotated pairs;
 *   kv    : for each block k of 64 dims in 0..447, amax = max |y|;
 *           e = least integer with amax <= 448 * 2^e, clamped to [-127, 127]
 *           (amax == 0 gives -127); code_j = E4M3(y_j * 2^-e) rounded to
 *           nearest even (e4m3fn, subnormals kept, sign kept); scale byte e+127;
 *           rope bytes = bf16 of the rotated values. */
int qkv_prep_run(qkv_prep_t h, const qkv_prep_args *args, void *stream);

/* Read slots back out of an FP8 + UE8M0 cache (the reader of this cache; the
 * 1Cat-vLLM PR 1280 page, change 5, names it dequantize_and_gather_k_cache).
 * Enqueue on `stream` and return.  Row i of out: dims 0..447 are
 * code * 2^(scale byte - 127) of their 64-dim block, for any scale byte 0..255
 * (exact in fp32, except that values of 2^128 and above, which only byte 255
 * reaches, are +-infinity; E4M3 NaN codes give NaN; the bf16 output is the fp32
 * value rounded to nearest even), dims 448..511 the stored bf16 rope values.
 * The operator itself never writes byte 255 (its exponents stop at 127).  Uses the handle's device and block_size; the handle must have
 * been created with kv_store = QKV_PREP_KV_FP8 (else QKV_PREP_ERR_UNSUPPORTED).
 * Limits: n < 2^26 and num_blocks * B < 2^31 (else QKV_PREP_ERR_UNSUPPORTED).
 * Argument errors are reported as for qkv_prep_run, with nothing launched.
 * Like qkv_prep_run, it allocates nothing and enqueues only its kernel. */
int qkv_prep_gather(qkv_prep_t h, const qkv_prep_gather_args *args, void *stream);

/* Release a handle.  NULL is a no-op.  Returns QKV_PREP_OK. */
int qkv_prep_destroy(qkv_prep_t h);

/* 1 if the kernel implements this shape (head_dim 512, rope_dim 64, H >= 1),
 * else 0.  A support gate in the manner of the rocm-aiter PR 1 page ("Technical
 * Details": a fixed-shape kernel exposes is_supported so that a caller serving
 * other shapes routes them to another kernel instead of tripping a check).
 * Pure host code; needs no device. */
int qkv_prep_supported(int32_t num_heads, int32_t head_dim, int32_t rope_dim);

/* The launch qkv_prep_run would use for num_tokens tokens with config cfg on
 * a device with num_cus compute units (256 on MI355X).  Pure host code: needs
 * no device, so the launch heuristic can be inspected anywhere.  The current
 * heuristic, for T tokens of H heads and q = T * H rows, as (q rows per
 * wavefront, wavefronts per workgroup, kv tokens per kv wavefront):
 *   q >= 2^16:  (2, 2, 4) with 2 <= H <= 56 and T >= 2^14, else (1, 1, 4);
 *   else q >= 49152, or q >= 2^15 with T > 4096, or q >= 24576 with
 *               T > 8192:  (1, 1, 4);
 *   else q >= 2^15 with T >= 2048:  (2, 2, 2);
 *   else T >= 3072, or T >= 2048 with H odd:  (1, 1, 2) when q >= 2^14 or
 *               T > 8192, else (1, 1, 1);
 *   else (2, 1, 1), and (1, 1, 1) for H = 1.
 * The kv workgroups come first in the grid, except with two heads and four kv
 * tokens per wavefront from 2^18 q rows, where they are spread over the first
 * 55-75% of it (out->kv_period).
 * A field forced in cfg replaces its part; the workgroup width then follows
 * the q rows per wavefront in use.  The heuristic does not depend on num_cus;
 * the argument keeps the signature stable for a device-dependent one.
 * Returns QKV_PREP_ERR_INVALID_ARG for a NULL out or num_tokens < 0, and
 * QKV_PREP_ERR_UNSUPPORTED when num_tokens * num_heads >= 2^31 (the limit of
 * qkv_prep_run). */
int qkv_prep_launch_shape(const qkv_prep_config *cfg, int32_t num_cus, int64_t num_tokens,
                          qkv_prep_launch *out);

/* The argument check qkv_prep_run performs, without a handle, device or
 * launch: returns QKV_PREP_OK or the error code run would return for these
 * arguments under cfg.  Pure host code. */
int qkv_prep_validate(const qkv_prep_config *cfg, const qkv_prep_args *args);

/* Static, NUL-terminated description of a return code. */
const char *qkv_prep_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* QKV_PREP_H */
