/* A C99 consumer of the library: no Python, no torch.  It includes only the
 * public headers and the HIP runtime's C API, allocates device memory, runs
 * qkv_prep_run and qkv_prep_gather on a small ragged case (37 tokens x 12
 * heads, 16-slot blocks, skipped and out-of-range slots, a poisoned cache) and
 * compares q, the whole cache and the gathered rows with the oracle's C
 * entry points (test infrastructure, compiled into this test program) byte
 * for byte.  Then it captures the same two calls into a HIP graph on a stream
 * of its own and replays the graph three times over freshly uploaded inputs,
 * each replay compared the same way: the calls allocate nothing and issue no
 * memset, so a C caller can capture them.  Last, qkv_prep_mxfp8_norm_quant on
 * 130 rows of hidden 640 (a ragged 128-row tile and a partial 512-group) with
 * the residual in and out: codes, the whole poisoned scale buffer and the
 * residual output against the oracle.  Exit status 0 = bit-exact; the last
 * line printed says which part differed otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "qkv_prep.h"
#include "qkv_prep_mxfp8.h"

/* The oracle (oracle/qkv_oracle.c). */
int orc_qkv_prep(int64_t num_tokens, int32_t num_heads, const uint16_t *q_in, uint16_t *q_out,
                 const uint16_t *kv, const uint16_t *q_w, const uint16_t *kv_w, const int64_t *positions,
                 const float *cos_sin, int64_t max_position, const int64_t *slot_mapping, uint8_t *cache,
                 int64_t num_blocks, int32_t block_size, float eps, int nthreads);
void orc_gather_dequant(const uint8_t *cache, int64_t num_blocks, int32_t block_size, const int64_t *slots,
                        int64_t n, float *out);
int orc_mxfp8_norm_quant(int64_t m, int64_t hidden, const uint16_t *x, const uint16_t *residual,
                         uint16_t *residual_out, const uint16_t *gamma, float eps, uint8_t *quant_out,
                         uint8_t *scale_out);

enum { T = 37, H = 12, B = 16, NB = 5, P = 1000, D = 512 };

static uint64_t state = 0x5DEECE66Dull;
static uint64_t next(void) /* splitmix64 */
{
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* A random bf16 bit pattern of magnitude 2^-7 .. 2^4 (any finite value is a
 * valid input; these are just not extreme). */
static uint16_t rand_bf16(void)
{
    const uint64_t r = next();
    return (uint16_t)(((r & 1) << 15) | ((120 + (r >> 1) % 12) << 7) | ((r >> 8) & 0x7f));
}

#define CHECK_HIP(x)                                                                     \
    do {                                                                                 \
        if ((x) != hipSuccess) {                                                         \
            printf("HIP call failed at line %d\n", __LINE__);                            \
            return 2;                                                                    \
        }                                                                                \
    } while (0)

/* The MXFP8 operator from C: 0 = bit-exact, 1 = a part differs, 2 = a call failed. */
enum { MXM = 130, MXH = 640 };

static int run_mxfp8(void)
{
    static uint16_t x[MXM * MXH], r[MXM * MXH], gamma[MXH], res_out[MXM * MXH], res_ref[MXM * MXH];
    static uint8_t codes[MXM * MXH], codes_ref[MXM * MXH];
    const int64_t ns = qkv_prep_mxfp8_scale_bytes(MXM, MXH);
    size_t i;
    if (ns <= 0) {
        printf("qkv_prep_mxfp8_scale_bytes failed\n");
        return 2;
    }
    uint8_t *scales = (uint8_t *)malloc((size_t)ns), *scales_ref = (uint8_t *)malloc((size_t)ns);
    if (!scales || !scales_ref)
        return 2;
    for (i = 0; i < MXM * MXH; ++i) {
        x[i] = rand_bf16();
        r[i] = rand_bf16();
    }
    for (i = 0; i < MXH; ++i)
        gamma[i] = (uint16_t)(rand_bf16() & 0xbfff);      /* |gamma| < 2 */
    void *dx, *dr, *dg, *dres, *dcodes, *dscales;
    CHECK_HIP(hipMalloc(&dx, sizeof(x)));
    CHECK_HIP(hipMalloc(&dr, sizeof(r)));
    CHECK_HIP(hipMalloc(&dg, sizeof(gamma)));
    CHECK_HIP(hipMalloc(&dres, sizeof(res_out)));
    CHECK_HIP(hipMalloc(&dcodes, sizeof(codes)));
    CHECK_HIP(hipMalloc(&dscales, (size_t)ns));
    CHECK_HIP(hipMemcpy(dx, x, sizeof(x), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dr, r, sizeof(r), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dg, gamma, sizeof(gamma), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(dscales, 0xee, (size_t)ns));     /* poison: every byte must be written */
    CHECK_HIP(hipMemset(dcodes, 0xee, sizeof(codes)));
    qkv_prep_mxfp8_args a;
    memset(&a, 0, sizeof(a));
    a.x = dx;
    a.residual = dr;
    a.residual_out = dres;
    a.gamma = dg;
    a.quant_out = dcodes;
    a.scale_out = dscales;
    a.m = MXM;
    a.hidden = MXH;
    a.eps = 1e-6f;
    const int rc = qkv_prep_mxfp8_norm_quant(&a, 0, NULL);
    if (rc != QKV_PREP_OK) {
        printf("qkv_prep_mxfp8_norm_quant: %s\n", qkv_prep_strerror(rc));
        return 2;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(codes, dcodes, sizeof(codes), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(scales, dscales, (size_t)ns, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(res_out, dres, sizeof(res_out), hipMemcpyDeviceToHost));
    if (orc_mxfp8_norm_quant(MXM, MXH, x, r, res_ref, gamma, 1e-6f, codes_ref, scales_ref) != 0) {
        printf("oracle rejected the MXFP8 case\n");
        return 2;
    }
    int bad = 0;
    if (memcmp(codes, codes_ref, sizeof(codes)) != 0) {
        printf("mxfp8: codes differ\n");
        bad = 1;
    } else if (memcmp(scales, scales_ref, (size_t)ns) != 0) {
        printf("mxfp8: scale bytes differ\n");
        bad = 1;
    } else if (memcmp(res_out, res_ref, sizeof(res_out)) != 0) {
        printf("mxfp8: residual output differs\n");
        bad = 1;
    }
    hipFree(dx); hipFree(dr); hipFree(dg); hipFree(dres); hipFree(dcodes); hipFree(dscales);
    free(scales);
    free(scales_ref);
    return bad;
}

/* Nonzero (after printing which part) when a result differs from the oracle. */
static int compare(const char *what, const void *q_out, const void *q_ref, size_t qn, const void *cache_out,
                   const void *cache_ref, size_t cn, const void *rows, const void *rows_ref, size_t rn)
{
    if (memcmp(q_out, q_ref, qn) != 0) {
        printf("c consumer (%s): q differs from the oracle\n", what);
        return 1;
    }
    if (memcmp(cache_out, cache_ref, cn) != 0) {
        printf("c consumer (%s): cache differs from the oracle\n", what);
        return 1;
    }
    if (memcmp(rows, rows_ref, rn) != 0) {
        printf("c consumer (%s): gathered rows differ from the oracle\n", what);
        return 1;
    }
    return 0;
}

int main(void)
{
    static uint16_t q[T * H * D], q_out[T * H * D], q_ref[T * H * D], kv[T * D], qw[D], kvw[D];
    static int64_t pos[T], slots[T + 2];
    static float cs[P * 64], rows[(T + 2) * D], rows_ref[(T + 2) * D];
    static uint8_t cache[NB * B * 584], cache_out[NB * B * 584], cache_ref[NB * B * 584];
    const size_t qn = sizeof(q), kvn = sizeof(kv), csn = sizeof(cs), cn = sizeof(cache);
    int i;

    for (i = 0; i < T * H * D; ++i)
        q[i] = rand_bf16();
    for (i = 0; i < T * D; ++i)
        kv[i] = rand_bf16();
    for (i = 0; i < D; ++i) {
        qw[i] = (uint16_t)(0x3F80 + (int)(next() % 33) - 16); /* bf16 near 1.0 */
        kvw[i] = (uint16_t)(0x3F80 + (int)(next() % 33) - 16);
    }
    for (i = 0; i < P * 64; ++i)
        cs[i] = (float)((double)(next() >> 11) / 9007199254740992.0 * 2.0 - 1.0);
    for (i = 0; i < T; ++i) {
        pos[i] = (int64_t)(next() % P);
        slots[i] = (int64_t)((i * 37 + 11) % (NB * B)); /* distinct: 37 is coprime to 80 */
    }
    slots[3] = -1;
    slots[20] = NB * B;      /* at capacity: skipped */
    slots[T] = -5;           /* two more rows for the reader */
    slots[T + 1] = 7;
    for (i = 0; i < (int)cn; ++i)
        cache[i] = (uint8_t)next();

    void *dq, *dkv, *dqw, *dkvw, *dpos, *dcs, *dslots, *dcache, *drows;
    CHECK_HIP(hipMalloc(&dq, qn));
    CHECK_HIP(hipMalloc(&dkv, kvn));
    CHECK_HIP(hipMalloc(&dqw, sizeof(qw)));
    CHECK_HIP(hipMalloc(&dkvw, sizeof(kvw)));
    CHECK_HIP(hipMalloc(&dpos, sizeof(pos)));
    CHECK_HIP(hipMalloc(&dcs, csn));
    CHECK_HIP(hipMalloc(&dslots, sizeof(slots)));
    CHECK_HIP(hipMalloc(&dcache, cn));
    CHECK_HIP(hipMalloc(&drows, sizeof(rows)));
    CHECK_HIP(hipMemcpy(dq, q, qn, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dkv, kv, kvn, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dqw, qw, sizeof(qw), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dkvw, kvw, sizeof(kvw), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dpos, pos, sizeof(pos), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dcs, cs, csn, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dslots, slots, sizeof(slots), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dcache, cache, cn, hipMemcpyHostToDevice));

    qkv_prep_config cfg;
    memset(&cfg, 0, sizeof(cfg));
    cfg.num_heads = H;
    cfg.head_dim = D;
    cfg.rope_dim = 64;
    cfg.block_size = B;
    cfg.eps = 1e-6f;
    cfg.kv_store = QKV_PREP_KV_FP8;
    qkv_prep_t h = NULL;
    int rc = qkv_prep_create(&cfg, 0, &h);
    if (rc != QKV_PREP_OK) {
        printf("qkv_prep_create: %s\n", qkv_prep_strerror(rc));
        return 2;
    }
    qkv_prep_args a;
    memset(&a, 0, sizeof(a));
    a.q = dq;
    a.kv = dkv;
    a.q_norm_w = dqw;
    a.kv_norm_w = dkvw;
    a.positions = (const int64_t *)dpos;
    a.cos_sin = (const float *)dcs;
    a.max_position = P;
    a.slot_mapping = (const int64_t *)dslots;
    a.kv_cache = dcache;
    a.num_blocks = NB;
    a.num_tokens = T;
    rc = qkv_prep_run(h, &a, NULL);
    if (rc != QKV_PREP_OK) {
        printf("qkv_prep_run: %s\n", qkv_prep_strerror(rc));
        return 2;
    }
    qkv_prep_gather_args g;
    memset(&g, 0, sizeof(g));
    g.kv_cache = dcache;
    g.num_blocks = NB;
    g.slots = (const int64_t *)dslots;
    g.n = T + 2;
    g.out = drows;
    g.out_dtype = QKV_PREP_OUT_F32;
    rc = qkv_prep_gather(h, &g, NULL);
    if (rc != QKV_PREP_OK) {
        printf("qkv_prep_gather: %s\n", qkv_prep_strerror(rc));
        return 2;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(q_out, dq, qn, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(cache_out, dcache, cn, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(rows, drows, sizeof(rows), hipMemcpyDeviceToHost));

    memcpy(cache_ref, cache, cn);
    if (orc_qkv_prep(T, H, q, q_ref, kv, qw, kvw, pos, cs, P, slots, cache_ref, NB, B, 1e-6f, 1) != 0) {
        printf("oracle rejected the case\n");
        return 2;
    }
    orc_gather_dequant(cache_ref, NB, B, slots, T + 2, rows_ref);
    if (compare("eager", q_out, q_ref, qn, cache_out, cache_ref, cn, rows, rows_ref, sizeof(rows)))
        return 1;

    /* The same two calls captured into a graph, replayed over fresh inputs. */
    hipStream_t st;
    hipGraph_t graph;
    hipGraphExec_t exec;
    CHECK_HIP(hipStreamCreate(&st));
    CHECK_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
    const int rc_run = qkv_prep_run(h, &a, st);
    const int rc_gather = qkv_prep_gather(h, &g, st);
    CHECK_HIP(hipStreamEndCapture(st, &graph));
    if (rc_run != QKV_PREP_OK || rc_gather != QKV_PREP_OK) {
        printf("capture: %s / %s\n", qkv_prep_strerror(rc_run), qkv_prep_strerror(rc_gather));
        return 2;
    }
    CHECK_HIP(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));
    for (i = 0; i < 3; ++i) {
        CHECK_HIP(hipMemcpy(dq, q, qn, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(dcache, cache, cn, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemset(drows, 0x7f, sizeof(rows)));
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipGraphLaunch(exec, st));
        CHECK_HIP(hipStreamSynchronize(st));
        CHECK_HIP(hipMemcpy(q_out, dq, qn, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(cache_out, dcache, cn, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(rows, drows, sizeof(rows), hipMemcpyDeviceToHost));
        if (compare("graph replay", q_out, q_ref, qn, cache_out, cache_ref, cn, rows, rows_ref, sizeof(rows)))
            return 1;
    }
    CHECK_HIP(hipGraphExecDestroy(exec));
    CHECK_HIP(hipGraphDestroy(graph));
    CHECK_HIP(hipStreamDestroy(st));
    qkv_prep_destroy(h);
    hipFree(dq); hipFree(dkv); hipFree(dqw); hipFree(dkvw); hipFree(dpos);
    hipFree(dcs); hipFree(dslots); hipFree(dcache); hipFree(drows);
    const int mx = run_mxfp8();
    if (mx != 0)
        return mx;
    printf("c consumer: q, cache and gathered rows bit-exact, eager and 3 graph replays (%d tokens x %d heads); "
           "MXFP8 codes, scales and residual bit-exact (%d x %d)\n", T, H, MXM, MXH);
    return 0;
}
