// Host side of the qkv_prep C ABI: argument checks, the launch-shape
// heuristic and the launch.  Declarations and contracts: include/qkv_prep.h.
#include "qkv_prep.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <new>

#include "qkv_prep_gather.h"
#include "qkv_prep_host.h"
#include "qkv_prep_internal.h"
#include "qkv_prep_launch.h"

struct qkv_prep {
    qkv_prep_config cfg;
    int device;
    int num_cus;
    bool sync;  // QKV_PREP_SYNC=1: wait for the stream inside run
    bool log;   // QKV_PREP_LOG=1: print a launch shape to stderr when it changes
    // The last launch shape printed (a packed key; ~0 = none yet).  Atomic so
    // that concurrent calls on one handle stay safe.
    std::atomic<uint64_t> logged{~0ull};
};

namespace {

using qkvp::aligned;
using qkvp::DeviceScope;
using qkvp::env_flag;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Launch result, then (with QKV_PREP_SYNC=1) the stream's.
int finish(const qkv_prep *h, hipError_t launched, hipStream_t st)
{
    if (launched != hipSuccess)
        return QKV_PREP_ERR_LAUNCH;
    if (h->sync && hipStreamSynchronize(st) != hipSuccess)
        return QKV_PREP_ERR_DEVICE;
    return QKV_PREP_OK;
}

// Where the kv workgroups sit in the grid.  By default they come first: the
// kv rows run as a latency-bound burst while the q stream starts behind them.
// With two heads per q wavefront and four kv tokens per kv wavefront, from
// 2^18 q rows, they are spread instead over the first 55-75% of the grid, one
// every P workgroups (P = floor(3N / 4K) for N workgroups of which K are kv,
// rounded down to an odd number so that the kv workgroups fall on every XCD
// in turn; none when that leaves P < 3).
// Measured on MI355X (eight interleaved rounds, one process), against kv
// first: 1.6-5.2% faster at all 15 such sizes tried, from 131072x2 and
// 32768x8 to 524288x2 and 131072x16 (131072x16: 709.8 -> 672.7 us; 131072x8:
// 377.3 -> 361.3 us).  Spreading over the whole grid ranged from 4.9% faster
// to 2.2% slower there, and over its first half from 0 to 3.5% faster.
// Elsewhere kv first stays: spread, the one-row shape lost 1.6-4.7% from
// 65536x24 to 131072x32 and 1-8% on the large workloads with 64 and 128
// heads, and batches below 2^18 q rows lost up to 25%.
int64_t kv_spread(const qkvp::LaunchShape &s, int64_t q_rows)
{
    if (s.rows_per_wave != 2 || s.kv_per_wave != 4 || q_rows < ((int64_t)1 << 18))
        return 0;
    const int64_t n = s.kv_blocks + s.q_blocks;
    int64_t p = 3 * n / (4 * s.kv_blocks);
    if (p % 2 == 0)
        p -= 1;
    return p >= 3 && n < ((int64_t)1 << 31) ? p : 0;
}

// Launch shape for T tokens of H heads (q_rows = T * H).  Chosen from the
// committed sweep (bench.py --mode sweep: each forced shape, 30 back-to-back
// launches, best of three interleaved rounds, after warming the chip), run on
// MI355X over a grid of 92 sizes (T 512 to 131072, H 1 to 128, 2^12 to 2^17
// q rows) twice, and checked on 46 sizes the rule was not fitted on.
//
// From 2^16 q rows:
//  * one q row per wavefront, with system-scope stores (2048x64: 41.7
//    against 42.5 us for two heads), except with at most 56 heads from 2^14
//    tokens, where two consecutive heads of one token per wavefront (the
//    token's position, cos/sin row and q weight loaded once for both rows)
//    are faster: 2-7% with at most 16 heads (32768x8: 94.6 against 101.1
//    us), and 0.8-4.4% with 17-56 heads, where the q rows pass 2^18 and the
//    kv workgroups are spread (kv_spread; 32768x20: 210.5 against 220.1 us,
//    65536x24: 497.6 against 516.8).  With 57-63 heads the two tie or one
//    row wins (16384x63: 2% for one row), and from 64 heads one row wins or
//    ties (32768x64: 0.5%);
//  * four consecutive tokens' kv rows per kv wavefront, their loads issued
//    together (the kv wavefronts run first, as a latency-bound burst;
//    2048x32: 22.3 against 23.3 us);
//  * two wavefronts per workgroup with the two-heads shape (0.8-2.6% faster
//    at all eight sizes from 16384x8 to 65536x16; 32768x8: 94.3 against
//    95.9 us);
//  * a grid past what one dispatch takes (2^32 work-items, from about 2^26 q
//    rows) is split into consecutive dispatches rather than narrowed to more
//    heads per wavefront: at 600000x128 one row per wavefront over two
//    dispatches keeps the large-batch rate, where two heads per wavefront
//    ran at 6.30 TB/s (and four, at 1100000x128, at 6.16).
// Below 2^16 q rows the kv rows are a large share of the work when heads
// are few, and the shape follows the token count as much as the row count:
//  * one row and four kv tokens per wavefront from 49152 q rows, from 2^15
//    with more than 4096 tokens, and from 24576 with more than 8192
//    (16384x3: 22.5 against 24.9 us for two heads and two kv tokens;
//    24576x1: 18.8 against 22.1 for one kv token);
//  * else, from 2^15 q rows with at least 2048 tokens: two heads per
//    wavefront, two kv tokens, two wavefronts per workgroup (4096x8: 13.5
//    against 14.2 us for one row and four kv tokens);
//  * else, from 3072 tokens, or from 2048 with an odd head count (where the
//    last of a token's two-heads wavefronts is half empty): one row per
//    wavefront, and two kv tokens from 2^14 q rows or above 8192 tokens, one
//    below (8192x3: 12.6 against 15.3 us for two heads; 2048x7: 8.1
//    against 8.8);
//  * else two heads per wavefront and one kv token (1024x16: 7.2 against
//    8.1 us for one row).
// Over both grid runs and the held-out sizes the rule averages 0.5-0.9%
// above the fastest shape per size and 6.2% at most; the rule it replaced
// averaged 3.2-5.6% above, and up to 22%.  Four heads per wavefront never
// won in the sweeps over every shape, and four wavefronts per workgroup win
// by 1.6% at most.
//  * convert: the gfx950 conversion instructions (bit-identical to the integer
//    rounding, which the tests check on every workload).
// A forced field (non-zero in the config) overrides its part; the workgroup
// width then still follows the q rows per wavefront in use, and the place of
// the kv workgroups in the grid follows the shape in use (kv_spread).
qkvp::LaunchShape choose_shape(const qkv_prep_config &c, int num_cus, int64_t T)
{
    (void)num_cus;
    qkvp::LaunchShape s;
    const int64_t H = c.num_heads;
    const int64_t q_rows = T * H;
    s.convert = c.convert ? c.convert : 2;
    int rows, kv;
    if (q_rows >= ((int64_t)1 << 16)) {
        rows = H > 1 && H <= 56 && T >= ((int64_t)1 << 14) ? 2 : 1;
        kv = 4;
    } else {
        const int64_t one_row_four_kv = T > 8192 ? 3 << 13 : T > 4096 ? 1 << 15 : 3 << 14;
        if (q_rows >= one_row_four_kv) {
            rows = 1;
            kv = 4;
        } else if (q_rows >= ((int64_t)1 << 15) && T >= 2048) {
            rows = H > 1 ? 2 : 1;
            kv = 2;
        } else if (T >= 3072 || (T >= 2048 && H % 2 == 1)) {
            rows = 1;
            kv = q_rows >= ((int64_t)1 << 14) || T > 8192 ? 2 : 1;
        } else {
            rows = H > 1 ? 2 : 1;
            kv = 1;
        }
    }
    s.rows_per_wave = c.rows_per_wave ? c.rows_per_wave : rows;
    s.kv_per_wave = c.kv_per_wave ? c.kv_per_wave : kv;
    // two wavefronts per workgroup with the two-heads shape wherever the
    // rule takes several kv tokens per wavefront
    s.waves_per_block = c.waves_per_block ? c.waves_per_block : s.rows_per_wave == 2 && kv >= 2 ? 2 : 1;
    s.kv_blocks = ceil_div(T, (int64_t)s.kv_per_wave * s.waves_per_block);
    // q wavefronts: T * ceil(H / U) (U heads of one token per wavefront)
    s.q_blocks = ceil_div(T * ceil_div(c.num_heads, s.rows_per_wave), s.waves_per_block);
    s.kv_period = kv_spread(s, q_rows);
    return s;
}

// Row indices are 32-bit inside the kernel: T * H must stay below 2^31.  Also
// keeps the launch-shape arithmetic (T * H, T * ceil(H / U)) inside int64.
bool rows_fit(const qkv_prep_config &c, int64_t T)
{
    return T <= (int64_t)0x7fffffff / c.num_heads;
}

int check_config(const qkv_prep_config *cfg)
{
    if (!cfg)
        return QKV_PREP_ERR_INVALID_ARG;
    if (cfg->num_heads < 1 || cfg->block_size < 1 || !(cfg->eps >= 0.0f) || cfg->eps > 3.4e38f)
        return QKV_PREP_ERR_INVALID_ARG;
    if (cfg->rows_per_wave != 0 && cfg->rows_per_wave != 1 && cfg->rows_per_wave != 2 &&
        cfg->rows_per_wave != 4)
        return QKV_PREP_ERR_INVALID_ARG;
    if (cfg->waves_per_block != 0 && cfg->waves_per_block != 1 && cfg->waves_per_block != 2 &&
        cfg->waves_per_block != 4 && cfg->waves_per_block != 8)
        return QKV_PREP_ERR_INVALID_ARG;
    if (cfg->convert < 0 || cfg->convert > 2)
        return QKV_PREP_ERR_INVALID_ARG;
    if (cfg->kv_store != QKV_PREP_KV_FP8 && cfg->kv_store != QKV_PREP_KV_BF16)
        return QKV_PREP_ERR_INVALID_ARG;
    if (cfg->kv_per_wave != 0 && cfg->kv_per_wave != 1 && cfg->kv_per_wave != 2 && cfg->kv_per_wave != 4)
        return QKV_PREP_ERR_INVALID_ARG;
    if (cfg->head_dim != qkvp::kHeadDim || cfg->rope_dim != qkvp::kRopeDim)
        return QKV_PREP_ERR_UNSUPPORTED;
    return QKV_PREP_OK;
}

// Everything qkv_prep_run checks before it touches the device.
int check_args(const qkv_prep_config &c, const qkv_prep_args *a)
{
    if (!a)
        return QKV_PREP_ERR_INVALID_ARG;
    const int64_t T = a->num_tokens;
    if (T < 0 || a->num_blocks < 0 || a->max_position < 1)
        return QKV_PREP_ERR_INVALID_ARG;
    if (T == 0)
        return QKV_PREP_OK;
    if (!a->q || !a->kv || !a->kv_norm_w || !a->positions || !a->cos_sin || !a->slot_mapping ||
        (a->num_blocks > 0 && !a->kv_cache))
        return QKV_PREP_ERR_INVALID_ARG;
    if (!aligned(a->q, 16) || !aligned(a->kv, 16) || !aligned(a->kv_norm_w, 16) ||
        (a->q_norm_w && !aligned(a->q_norm_w, 16)) || !aligned(a->cos_sin, 16) ||
        (a->kv_cache && !aligned(a->kv_cache, 16)) || !aligned(a->positions, 8) ||
        !aligned(a->slot_mapping, 8))
        return QKV_PREP_ERR_MISALIGNED;
    const int64_t B = c.block_size;
    // Row and slot indices are 32-bit inside the kernel; addresses are 64-bit.
    if (!rows_fit(c, T) || a->num_blocks > (int64_t)0x7fffffff / B ||
        a->max_position > ((int64_t)1 << 40))
        return QKV_PREP_ERR_UNSUPPORTED;
    return QKV_PREP_OK;    // any grid: one past what a dispatch takes is split (launch_qkv_prep)
}

int check_gather(const qkv_prep_config &c, const qkv_prep_gather_args *a)
{
    if (!a)
        return QKV_PREP_ERR_INVALID_ARG;
    if (c.kv_store != QKV_PREP_KV_FP8)
        return QKV_PREP_ERR_UNSUPPORTED;
    if (a->n < 0 || a->num_blocks < 0 ||
        (a->out_dtype != QKV_PREP_OUT_F32 && a->out_dtype != QKV_PREP_OUT_BF16))
        return QKV_PREP_ERR_INVALID_ARG;
    if (a->n == 0)
        return QKV_PREP_OK;
    if (!a->slots || !a->out || (a->num_blocks > 0 && !a->kv_cache))
        return QKV_PREP_ERR_INVALID_ARG;
    if ((a->kv_cache && !aligned(a->kv_cache, 16)) || !aligned(a->out, 16) || !aligned(a->slots, 8))
        return QKV_PREP_ERR_MISALIGNED;
    if (a->num_blocks > (int64_t)0x7fffffff / c.block_size || a->n >= ((int64_t)1 << 26))
        return QKV_PREP_ERR_UNSUPPORTED;
    return QKV_PREP_OK;
}

}  // namespace

extern "C" {

const char *qkv_prep_strerror(int code)
{
    switch (code) {
    case QKV_PREP_OK: return "ok";
    case QKV_PREP_ERR_INVALID_ARG: return "invalid argument";
    case QKV_PREP_ERR_UNSUPPORTED: return "unsupported shape";
    case QKV_PREP_ERR_MISALIGNED: return "misaligned pointer";
    case QKV_PREP_ERR_NO_DEVICE: return "no such HIP device";
    case QKV_PREP_ERR_LAUNCH: return "kernel launch failed";
    case QKV_PREP_ERR_DEVICE: return "device error during the call";
    default: return "unknown qkv_prep error";
    }
}

int qkv_prep_supported(int32_t num_heads, int32_t head_dim, int32_t rope_dim)
{
    return num_heads >= 1 && head_dim == qkvp::kHeadDim && rope_dim == qkvp::kRopeDim;
}

int qkv_prep_create(const qkv_prep_config *cfg, int device, qkv_prep_t *out)
{
    if (!out)
        return QKV_PREP_ERR_INVALID_ARG;
    const int rc = check_config(cfg);
    if (rc != QKV_PREP_OK)
        return rc;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return QKV_PREP_ERR_NO_DEVICE;
    }
    if (device < 0 || device >= count)
        return QKV_PREP_ERR_NO_DEVICE;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
        (void)hipGetLastError();
        return QKV_PREP_ERR_NO_DEVICE;
    }
    qkv_prep *h = new (std::nothrow) qkv_prep;
    if (!h)
        return QKV_PREP_ERR_INVALID_ARG;
    h->cfg = *cfg;
    h->device = device;
    h->num_cus = cus;
    h->sync = env_flag("QKV_PREP_SYNC");
    h->log = env_flag("QKV_PREP_LOG");
    *out = h;
    return QKV_PREP_OK;
}

int qkv_prep_destroy(qkv_prep_t h)
{
    delete h;
    return QKV_PREP_OK;
}

int qkv_prep_launch_shape(const qkv_prep_config *cfg, int32_t num_cus, int64_t num_tokens,
                          qkv_prep_launch *out)
{
    const int rc = check_config(cfg);
    if (rc != QKV_PREP_OK)
        return rc;
    if (!out || num_tokens < 0)
        return QKV_PREP_ERR_INVALID_ARG;
    if (!rows_fit(*cfg, num_tokens))
        return QKV_PREP_ERR_UNSUPPORTED;
    const qkvp::LaunchShape s = choose_shape(*cfg, num_cus, num_tokens);
    out->rows_per_wave = s.rows_per_wave;
    out->waves_per_block = s.waves_per_block;
    out->convert = s.convert;
    out->kv_per_wave = s.kv_per_wave;
    out->kv_blocks = num_tokens ? s.kv_blocks : 0;
    out->q_blocks = num_tokens ? s.q_blocks : 0;
    out->kv_period = num_tokens ? s.kv_period : 0;
    out->grid = out->kv_blocks + out->q_blocks;
    return QKV_PREP_OK;
}

int qkv_prep_validate(const qkv_prep_config *cfg, const qkv_prep_args *args)
{
    const int rc = check_config(cfg);
    return rc != QKV_PREP_OK ? rc : check_args(*cfg, args);
}

int qkv_prep_run(qkv_prep_t h, const qkv_prep_args *a, void *stream)
{
    if (!h)
        return QKV_PREP_ERR_INVALID_ARG;
    const int rc_args = check_args(h->cfg, a);
    if (rc_args != QKV_PREP_OK || a->num_tokens == 0)
        return rc_args;
    const int64_t T = a->num_tokens;
    const int64_t H = h->cfg.num_heads;
    const int64_t B = h->cfg.block_size;
    const qkvp::LaunchShape s = choose_shape(h->cfg, h->num_cus, T);

    qkvp::KernelArgs k{};
    k.q = static_cast<uint16_t *>(a->q);
    k.kv = static_cast<const uint16_t *>(a->kv);
    k.q_w = static_cast<const uint16_t *>(a->q_norm_w);
    k.kv_w = static_cast<const uint16_t *>(a->kv_norm_w);
    k.positions = a->positions;
    k.cos_sin = a->cos_sin;
    k.slot_mapping = a->slot_mapping;
    k.cache = static_cast<uint8_t *>(a->kv_cache);
    k.max_position = a->max_position;
    k.num_slots = a->num_blocks * B;
    k.q_rows = T * H;
    k.num_tokens = T;
    k.block_size = (uint32_t)B;
    k.kv_blocks = (uint32_t)s.kv_blocks;
    k.kv_per_wave = (uint32_t)s.kv_per_wave;
    k.heads = qkvp::make_fastdiv((uint32_t)H);
    k.blocks = qkvp::make_fastdiv((uint32_t)B);
    k.num_heads = (uint32_t)H;
    k.chunks = (uint32_t)ceil_div(H, s.rows_per_wave);
    k.chunk_div = qkvp::make_fastdiv(k.chunks);
    k.eps = h->cfg.eps;
    k.bf16_store = h->cfg.kv_store == QKV_PREP_KV_BF16;
    k.kv_period = (uint32_t)s.kv_period;
    if (s.kv_period)
        k.period_div = qkvp::make_fastdiv((uint32_t)s.kv_period);

    DeviceScope dev(h->device);
    if (!dev.ok())
        return QKV_PREP_ERR_NO_DEVICE;
    if (h->log) {
        const uint64_t key = (uint64_t)s.rows_per_wave | (uint64_t)s.kv_per_wave << 8 |
                             (uint64_t)s.waves_per_block << 16 | (uint64_t)s.convert << 24;
        if (h->logged.exchange(key, std::memory_order_relaxed) != key)
            std::fprintf(stderr,
                         "qkv_prep: launch shape rows/wave=%d kv/wave=%d waves/block=%d convert=%d "
                         "(first at T=%lld H=%lld, grid %lld+%lld workgroups)\n",
                         s.rows_per_wave, s.kv_per_wave, s.waves_per_block, s.convert, (long long)T,
                         (long long)H, (long long)s.kv_blocks, (long long)s.q_blocks);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish(h, qkvp::launch_qkv_prep(k, s, st), st);
}

int qkv_prep_gather(qkv_prep_t h, const qkv_prep_gather_args *a, void *stream)
{
    if (!h)
        return QKV_PREP_ERR_INVALID_ARG;
    const int rc_args = check_gather(h->cfg, a);
    if (rc_args != QKV_PREP_OK || a->n == 0)
        return rc_args;
    qkvp::GatherArgs g{};
    g.cache = static_cast<const uint8_t *>(a->kv_cache);
    g.slots = a->slots;
    g.out = a->out;
    g.num_slots = a->num_blocks * h->cfg.block_size;
    g.n = a->n;
    g.block_size = (uint32_t)h->cfg.block_size;
    g.blocks = qkvp::make_fastdiv((uint32_t)h->cfg.block_size);
    g.out_bf16 = a->out_dtype == QKV_PREP_OUT_BF16;
    DeviceScope dev(h->device);
    if (!dev.ok())
        return QKV_PREP_ERR_NO_DEVICE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish(h, qkvp::launch_gather(g, 1, st), st);
}

}  // extern "C"
