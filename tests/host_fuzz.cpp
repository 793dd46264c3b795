// Host-only fuzz of the C ABI, built with -fsanitize=address,undefined by
// tests/test_host_sanitized.py and linked with the host API only
// (qkv_prep_api.cpp, mxfp8_api.cpp).  The two
// kernel launchers are stubbed (they record what they were given), and the six
// HIP runtime calls the host API makes are defined here as a fake two-device
// runtime, so nothing touches a GPU and no HIP library is linked.
//  * Extreme and random configs and arguments go through qkv_prep_validate,
//    qkv_prep_launch_shape, qkv_prep_supported and qkv_prep_strerror.
//  * Handles are created on the fake devices and qkv_prep_run /
//    qkv_prep_gather are called with extreme and random arguments: run's code
//    must equal validate's, a launch happens exactly when the arguments are
//    valid and non-empty, the launch's arguments and grid must be consistent,
//    and the caller's current device must be restored after every call.
//  * qkv_prep_mxfp8_scale_bytes and qkv_prep_mxfp8_norm_quant on extreme and
//    random shapes, pointers and device indices: sizes against a 128-bit
//    reference, a launch exactly when valid, on the requested device with the
//    caller's device restored, the launch's rows and scale layout.
// Any undefined operation aborts the run; contract violations are counted.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "qkv_prep.h"
#include "qkv_prep_gather.h"
#include "qkv_prep_launch.h"
#include "qkv_prep_mxfp8.h"
#include "mxfp8_launch.h"

namespace {
int launches = 0, gathers = 0;
qkvp::KernelArgs last_k;
qkvp::LaunchShape last_s;
qkvp::GatherArgs last_g;
int fake_current = 0, fake_device_at_launch = -1;
}  // namespace

namespace qkvp {
hipError_t launch_qkv_prep(const KernelArgs &a, const LaunchShape &s, hipStream_t)
{
    ++launches;
    last_k = a;
    last_s = s;
    fake_device_at_launch = fake_current;
    return hipSuccess;
}
hipError_t launch_gather(const GatherArgs &a, int, hipStream_t)
{
    ++gathers;
    last_g = a;
    fake_device_at_launch = fake_current;
    return hipSuccess;
}
int mx_launches = 0;
MxArgs last_mx;
int mx_device_at_launch = -1;
hipError_t launch_mxfp8(const MxArgs &a, hipStream_t)
{
    ++mx_launches;
    last_mx = a;
    mx_device_at_launch = fake_current;
    return hipSuccess;
}
}  // namespace qkvp

// The fake runtime: two devices of 256 compute units.
extern "C" {
hipError_t hipGetDeviceCount(int *count)
{
    *count = 2;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t, int device)
{
    if (device < 0 || device > 1)
        return hipErrorInvalidDevice;
    *value = 256;
    return hipSuccess;
}
hipError_t hipGetDevice(int *device)
{
    *device = fake_current;
    return hipSuccess;
}
hipError_t hipSetDevice(int device)
{
    if (device < 0 || device > 1)
        return hipErrorInvalidDevice;
    fake_current = device;
    return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}

namespace {

uint64_t state = 0x243F6A8885A308D3ull;
uint64_t next()  // splitmix64
{
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int32_t pick32()
{
    static const int32_t v[] = {0, 1, -1, 2, 3, 4, 5, 7, 8, 16, 64, 128, 448, 512, 513, 1024,
                                std::numeric_limits<int32_t>::max(), std::numeric_limits<int32_t>::min()};
    return next() % 4 == 0 ? (int32_t)next() : v[next() % (sizeof(v) / sizeof(v[0]))];
}

int64_t pick64()
{
    static const int64_t v[] = {0, 1, -1, 2, 17, 4096, 131072, (int64_t)1 << 19, ((int64_t)1 << 31) - 1,
                                (int64_t)1 << 31, (int64_t)1 << 40, ((int64_t)1 << 40) + 1,
                                std::numeric_limits<int64_t>::max(), std::numeric_limits<int64_t>::min()};
    const uint64_t r = next() % 4;
    if (r == 0)
        return (int64_t)next();
    if (r == 1)
        return (int64_t)(next() % 100000);
    return v[next() % (sizeof(v) / sizeof(v[0]))];
}

float pick_eps()
{
    static const float v[] = {0.0f, 1e-6f, -1e-6f, 1.0f, 3.4e38f, std::numeric_limits<float>::infinity(),
                              std::numeric_limits<float>::quiet_NaN(), -0.0f};
    return v[next() % (sizeof(v) / sizeof(v[0]))];
}

// Fake device addresses (never dereferenced): mostly 16-byte aligned, else
// NULL, 8-byte aligned or odd.
void *pick_ptr()
{
    static const uintptr_t v[] = {0, 0x100008, 0x100001};
    if (next() % 8)
        return reinterpret_cast<void *>((uintptr_t)0x100000 + 16 * (next() % 4096));
    return reinterpret_cast<void *>(v[next() % (sizeof(v) / sizeof(v[0]))]);
}

int failures = 0;
void expect(bool ok, const char *what, long long i)
{
    if (!ok && failures++ < 20)
        std::fprintf(stderr, "contract violated at case %lld: %s\n", i, what);
}

}  // namespace

int main()
{
    const long long cases = 400000;
    long long ok_validate = 0, ok_shape = 0;
    for (long long i = 0; i < cases; ++i) {
        qkv_prep_config c;
        std::memset(&c, 0, sizeof(c));
        c.num_heads = next() % 3 ? (int32_t)(1 + next() % 256) : pick32();
        c.head_dim = next() % 8 ? 512 : pick32();
        c.rope_dim = next() % 8 ? 64 : pick32();
        c.block_size = next() % 3 ? (int32_t)(1 + next() % 256) : pick32();
        c.eps = pick_eps();
        c.rows_per_wave = next() % 2 ? 0 : pick32() % 6;
        c.waves_per_block = next() % 2 ? 0 : pick32() % 10;
        c.convert = next() % 2 ? 0 : pick32() % 4;
        c.kv_store = next() % 4 ? (int32_t)(next() % 2) : pick32();
        c.kv_per_wave = next() % 2 ? 0 : pick32() % 6;

        const int64_t T = next() % 2 ? (int64_t)(next() % 200000) : pick64();
        qkv_prep_launch sh;
        const int rs = qkv_prep_launch_shape(&c, (int32_t)(next() % 512), T, &sh);
        expect(rs >= 0 && rs <= 6, "launch_shape code", i);
        if (rs == QKV_PREP_OK) {
            ++ok_shape;
            expect(sh.grid == sh.kv_blocks + sh.q_blocks, "grid = kv + q", i);
            expect(sh.kv_blocks >= 0 && sh.q_blocks >= 0, "non-negative blocks", i);
            expect(sh.rows_per_wave == 1 || sh.rows_per_wave == 2 || sh.rows_per_wave == 4, "rows per wave", i);
            expect(sh.kv_per_wave == 1 || sh.kv_per_wave == 2 || sh.kv_per_wave == 4, "kv rows per wave", i);
            expect(T > 0 || sh.grid == 0, "empty batch launches nothing", i);
        }

        qkv_prep_args a;
        std::memset(&a, 0, sizeof(a));
        a.q = pick_ptr();
        a.kv = pick_ptr();
        a.q_norm_w = next() % 2 ? nullptr : pick_ptr();
        a.kv_norm_w = pick_ptr();
        a.positions = static_cast<const int64_t *>(pick_ptr());
        a.cos_sin = static_cast<const float *>(pick_ptr());
        a.max_position = next() % 2 ? (int64_t)(1 + next() % 200000) : pick64();
        a.slot_mapping = static_cast<const int64_t *>(pick_ptr());
        a.kv_cache = pick_ptr();
        a.num_blocks = next() % 2 ? (int64_t)(next() % 100000) : pick64();
        a.num_tokens = T;
        const int rv = qkv_prep_validate(&c, &a);
        expect(rv >= 0 && rv <= 6, "validate code", i);
        if (rv == QKV_PREP_OK && T > 0) {
            ++ok_validate;
            expect(rs == QKV_PREP_OK, "valid args have a launch shape", i);
            expect(sh.grid < ((int64_t)1 << 32) && sh.kv_blocks < ((int64_t)1 << 32),
                   "workgroup indices fit 32 bits", i);
            expect(T * (int64_t)c.num_heads <= 0x7fffffff, "row indices fit 31 bits", i);
            expect(std::isfinite(c.eps) && c.eps >= 0.0f, "eps finite and >= 0", i);
        }
        expect(qkv_prep_validate(nullptr, &a) == QKV_PREP_ERR_INVALID_ARG, "null cfg", i);
        expect(qkv_prep_validate(&c, nullptr) != QKV_PREP_OK || c.num_heads < 1, "null args", i);
        expect(qkv_prep_launch_shape(&c, 256, T, nullptr) != QKV_PREP_OK, "null out", i);
        const int sup = qkv_prep_supported(c.num_heads, c.head_dim, c.rope_dim);
        expect(sup == 0 || sup == 1, "supported is 0/1", i);
        expect(std::strlen(qkv_prep_strerror((int)next())) > 0, "strerror non-empty", i);
    }

    // Handles on the fake devices: run and gather against the contract.
    long long runs_ok = 0, gathers_ok = 0, spread_runs = 0;
    for (long long i = 0; i < 100000; ++i) {
        qkv_prep_config c;
        std::memset(&c, 0, sizeof(c));
        c.num_heads = next() % 4 ? (int32_t)(1 + next() % 160) : pick32();
        c.head_dim = 512;
        c.rope_dim = 64;
        c.block_size = next() % 4 ? (int32_t)(1 + next() % 128) : pick32();
        c.eps = next() % 8 ? 1e-6f : pick_eps();
        c.kv_store = (int32_t)(next() % 2);
        const int device = (int)(next() % 3) - (next() % 8 == 0);   // -1..2, mostly 0/1
        qkv_prep_t h = nullptr;
        const int rc = qkv_prep_create(&c, device, &h);
        const bool cfg_ok = c.num_heads >= 1 && c.block_size >= 1 && std::isfinite(c.eps) && c.eps >= 0.0f;
        expect((rc == QKV_PREP_OK) == (cfg_ok && device >= 0 && device <= 1), "create succeeds iff valid", i);
        expect((rc == QKV_PREP_OK) == (h != nullptr), "handle set only on success", i);
        if (rc != QKV_PREP_OK)
            continue;
        for (int r = 0; r < 4; ++r) {
            qkv_prep_args a;
            std::memset(&a, 0, sizeof(a));
            a.q = pick_ptr();
            a.kv = pick_ptr();
            a.q_norm_w = next() % 2 ? nullptr : pick_ptr();
            a.kv_norm_w = pick_ptr();
            a.positions = static_cast<const int64_t *>(pick_ptr());
            a.cos_sin = static_cast<const float *>(pick_ptr());
            a.max_position = next() % 2 ? (int64_t)(1 + next() % 200000) : pick64();
            a.slot_mapping = static_cast<const int64_t *>(pick_ptr());
            a.kv_cache = pick_ptr();
            a.num_blocks = next() % 2 ? (int64_t)(next() % 100000) : pick64();
            a.num_tokens = next() % 2 ? (int64_t)(next() % 300000) : pick64();
            const int caller = (int)(next() % 2);
            fake_current = caller;
            const int before = launches;
            const int rr = qkv_prep_run(h, &a, nullptr);
            const int rv = qkv_prep_validate(&c, &a);
            expect(rr == rv, "run code equals validate code", i);
            expect(fake_current == caller, "run restores the caller's device", i);
            const bool launched = launches != before;
            expect(launched == (rr == QKV_PREP_OK && a.num_tokens > 0), "launch iff valid and non-empty", i);
            if (launched) {
                ++runs_ok;
                expect(fake_device_at_launch == device, "launch on the handle's device", i);
                const qkvp::KernelArgs &k = last_k;
                expect(k.q == a.q && k.kv == a.kv && k.cache == a.kv_cache, "pointers passed through", i);
                expect(k.num_tokens == a.num_tokens && k.q_rows == a.num_tokens * c.num_heads, "sizes", i);
                expect(k.num_slots == a.num_blocks * c.block_size && k.num_slots < ((int64_t)1 << 31), "slots", i);
                expect(k.kv_blocks == (uint32_t)last_s.kv_blocks, "kv blocks", i);
                expect(k.chunks == (uint32_t)(((int64_t)c.num_heads + last_s.rows_per_wave - 1) / last_s.rows_per_wave),
                       "chunks per token", i);
                expect((int64_t)k.chunks * a.num_tokens < ((int64_t)1 << 31), "q wavefront index fits", i);
                {
                    const int64_t grid = last_s.kv_blocks + last_s.q_blocks;
                    const int64_t per = qkvp::max_blocks_per_launch(last_s.waves_per_block);
                    const int64_t n = qkvp::launches_for(grid, last_s.waves_per_block);
                    expect(per * 64 * last_s.waves_per_block < ((int64_t)1 << 32) &&
                               (per + 1) * 64 * last_s.waves_per_block >= ((int64_t)1 << 32),
                           "a dispatch holds as many workgroups as fit", i);
                    expect(n >= 1 && (n - 1) * per < grid && n * per >= grid, "dispatches cover the grid", i);
                }
                expect(last_s.q_blocks * last_s.waves_per_block >= a.num_tokens * (int64_t)k.chunks,
                       "every q wavefront has a slot in the grid", i);
                expect(last_s.kv_blocks * last_s.waves_per_block * last_s.kv_per_wave >= a.num_tokens,
                       "every kv row covered", i);
                expect(k.kv_per_wave == (uint32_t)last_s.kv_per_wave, "kv rows per wavefront", i);
                expect(k.bf16_store == (c.kv_store == QKV_PREP_KV_BF16), "store mode", i);
                expect(k.kv_period == (uint32_t)last_s.kv_period, "kv period passed through", i);
                if (last_s.kv_period != 0) {
                    // kv workgroup j at grid index j * P: only for two heads and
                    // four kv tokens per wavefront from 2^18 q rows; P odd (the kv
                    // workgroups fall on every XCD in turn) and >= 3; every kv
                    // workgroup inside a grid of fewer than 2^31 workgroups, where
                    // the kernel's fixed-point division by P is exact.
                    const int64_t p = last_s.kv_period;
                    const int64_t grid = last_s.kv_blocks + last_s.q_blocks;
                    ++spread_runs;
                    expect(last_s.rows_per_wave == 2 && last_s.kv_per_wave == 4 && k.q_rows >= ((int64_t)1 << 18),
                           "kv spread only for the large two-heads shape", i);
                    expect(p % 2 == 1 && p >= 3, "kv period odd and >= 3", i);
                    expect((last_s.kv_blocks - 1) * p < grid && grid < ((int64_t)1 << 31),
                           "kv workgroups inside the grid", i);
                    for (int64_t n : {(int64_t)0, p - 1, p, (last_s.kv_blocks - 1) * p, grid - 1,
                                      (int64_t)(next() % (uint64_t)grid)}) {
                        const uint32_t q32 = (uint32_t)((((uint64_t)(uint32_t)n * k.period_div.mul) >> 32) + (uint64_t)n)
                                             >> k.period_div.shift;
                        expect((int64_t)q32 == n / p, "fixed-point division by the kv period", i);
                    }
                } else {
                    expect(!(last_s.rows_per_wave == 2 && last_s.kv_per_wave == 4 && k.q_rows >= ((int64_t)1 << 18) &&
                             3 * (last_s.kv_blocks + last_s.q_blocks) / (4 * last_s.kv_blocks) >= 3),
                           "large two-heads batches spread their kv workgroups", i);
                }
            }

            qkv_prep_gather_args g;
            std::memset(&g, 0, sizeof(g));
            g.kv_cache = pick_ptr();
            g.num_blocks = next() % 2 ? (int64_t)(next() % 100000) : pick64();
            g.slots = static_cast<const int64_t *>(pick_ptr());
            g.n = next() % 2 ? (int64_t)(next() % 100000) : pick64();
            g.out = pick_ptr();
            g.out_dtype = next() % 8 ? (int32_t)(next() % 2) : pick32();
            fake_current = caller;
            const int gbefore = gathers;
            const int rg = qkv_prep_gather(h, &g, nullptr);
            expect(rg >= 0 && rg <= 6, "gather code", i);
            expect(fake_current == caller, "gather restores the caller's device", i);
            const bool glaunched = gathers != gbefore;
            expect(glaunched == (rg == QKV_PREP_OK && g.n > 0), "gather launch iff valid and non-empty", i);
            if (c.kv_store == QKV_PREP_KV_BF16)
                expect(rg == QKV_PREP_ERR_UNSUPPORTED || rg == QKV_PREP_ERR_INVALID_ARG, "bf16 handle has no reader", i);
            if (glaunched) {
                ++gathers_ok;
                expect(last_g.n == g.n && g.n < ((int64_t)1 << 26), "gather rows", i);
                for (int wpb : {1, 2, 4, 8})
                    for (int bf : {0, 1}) {
                        const qkvp::GatherGrid gg = qkvp::gather_grid(g.n, bf != 0, wpb);
                        const int rows = bf ? qkvp::kBf16Rows : qkvp::kF32Rows;
                        expect(gg.blocks * 64 * wpb < ((int64_t)1 << 32), "gather grid fits", i);
                        expect(gg.blocks * wpb * rows >= g.n, "gather grid covers every row", i);
                    }
                expect(last_g.num_slots == g.num_blocks * c.block_size && last_g.num_slots < ((int64_t)1 << 31),
                       "gather slots", i);
                expect(last_g.out_bf16 == (g.out_dtype == QKV_PREP_OUT_BF16), "gather dtype", i);
            }
        }
        expect(qkv_prep_destroy(h) == QKV_PREP_OK, "destroy", i);
    }
    expect(qkv_prep_destroy(nullptr) == QKV_PREP_OK, "destroy NULL", 0);
    expect(qkv_prep_run(nullptr, nullptr, nullptr) == QKV_PREP_ERR_INVALID_ARG, "run NULL handle", 0);
    expect(qkv_prep_gather(nullptr, nullptr, nullptr) == QKV_PREP_ERR_INVALID_ARG, "gather NULL handle", 0);

    // The MXFP8 entry points.
    long long mx_ok = 0;
    for (long long i = 0; i < 200000; ++i) {
        const int64_t m = next() % 2 ? (int64_t)(next() % 100000) : pick64();
        const int32_t hidden = next() % 2 ? (int32_t)(128 * (next() % 140)) : pick32();
        const int64_t sb = qkv_prep_mxfp8_scale_bytes(m, hidden);
        if (m < 0 || hidden <= 0 || hidden % 128) {
            expect(sb == -1, "scale bytes -1 for bad shapes", i);
        } else {
            const __int128 want = ((__int128)m + 127) / 128 * 128 * (hidden / 32);
            expect(want > INT64_MAX ? sb == -1 : (__int128)sb == want, "scale bytes value", i);
        }
        qkv_prep_mxfp8_args a;
        std::memset(&a, 0, sizeof(a));
        a.x = pick_ptr();
        a.residual = next() % 2 ? nullptr : pick_ptr();
        a.residual_out = next() % 2 ? nullptr : pick_ptr();
        a.gamma = pick_ptr();
        a.quant_out = pick_ptr();
        a.scale_out = pick_ptr();
        a.m = m;
        a.hidden = hidden;
        a.eps = next() % 4 ? 1e-6f : pick_eps();
        const int before = qkvp::mx_launches;
        static const int devices[] = {0, 1, 1, 0, -1, 2, std::numeric_limits<int>::min()};
        const int device = devices[next() % (sizeof(devices) / sizeof(devices[0]))];
        fake_current = (int)(next() % 2);
        const int caller_device = fake_current;
        const int rc = qkv_prep_mxfp8_norm_quant(&a, device, nullptr);
        expect(rc >= 0 && rc <= 6 && rc != QKV_PREP_ERR_DEVICE, "mxfp8 code", i);
        expect(fake_current == caller_device, "mxfp8 restores the caller's device", i);
        const bool launched = qkvp::mx_launches != before;
        expect(launched == (rc == QKV_PREP_OK && m > 0), "mxfp8 launch iff valid and non-empty", i);
        if (rc == QKV_PREP_ERR_NO_DEVICE)
            expect(device < 0 || device > 1, "mxfp8 no-device only for a missing device", i);
        if (launched) {
            ++mx_ok;
            expect(qkvp::mx_device_at_launch == device, "mxfp8 launches on the requested device", i);
            const qkvp::MxArgs &k = qkvp::last_mx;
            expect(hidden >= 128 && hidden <= 16384 && hidden % 128 == 0, "hidden supported", i);
            expect(k.chunks == hidden / 8, "chunks", i);
            expect((reinterpret_cast<uintptr_t>(k.scale_out) & 3) == 0, "scale words aligned", i);
            expect(k.rows_padded == (m + 127) / 128 * 128 && k.rows_padded < ((int64_t)1 << 31), "rows", i);
            expect(k.rows_padded * qkvp::mx_threads_per_row(hidden) < ((int64_t)1 << 32), "grid fits", i);
            expect(k.padded_cols == hidden / 32 && (int64_t)k.rows_padded * k.padded_cols == sb, "scale layout", i);
            expect(std::isfinite(k.eps) && k.eps >= 0.0f, "eps", i);
        }
    }
    expect(qkv_prep_mxfp8_norm_quant(nullptr, 0, nullptr) == QKV_PREP_ERR_INVALID_ARG, "mxfp8 NULL", 0);

    // The work-item limit at its edge, for workgroups of 64 (hidden 128),
    // 192 (hidden 1152: three groups, one per wavefront) and 1024 lanes
    // (hidden 16384): the largest padded row count that fits launches, one
    // more tile is refused.
    {
        static const struct { int32_t hidden; int64_t lanes; } edges[] = {{128, 64}, {1152, 192}, {16384, 1024}};
        for (const auto &e : edges) {
            expect(qkvp::mx_threads_per_row(e.hidden) == e.lanes, "workgroup size", e.hidden);
            const int64_t max_rows = (((int64_t)1 << 32) - 1) / e.lanes / 128 * 128;
            for (int64_t m : {max_rows, max_rows - 127, max_rows + 1}) {
                qkv_prep_mxfp8_args a;
                std::memset(&a, 0, sizeof(a));
                a.x = a.gamma = reinterpret_cast<const void *>(0x100000);
                a.quant_out = a.scale_out = reinterpret_cast<void *>(0x200000);
                a.m = m;
                a.hidden = e.hidden;
                a.eps = 1e-6f;
                const int rc = qkv_prep_mxfp8_norm_quant(&a, 0, nullptr);
                expect(rc == (m <= max_rows ? QKV_PREP_OK : QKV_PREP_ERR_UNSUPPORTED), "mxfp8 grid edge", m);
            }
        }
    }
    // The reader's grid at its row limit: the XCD padding would reach 2^32
    // work-items, so the plain order is kept; a little below it, it pads.
    {
        const qkvp::GatherGrid top = qkvp::gather_grid(((int64_t)1 << 26) - 1, false, 1);
        expect(top.xcd_chunk == 0 && top.blocks == ((int64_t)1 << 26) - 1, "reader grid at the limit", 0);
        const qkvp::GatherGrid below = qkvp::gather_grid(((int64_t)1 << 26) - 512, false, 1);
        expect(below.xcd_chunk == 64 && below.blocks == ((int64_t)1 << 26) - 512, "reader grid below the limit", 0);
        const qkvp::GatherGrid bf = qkvp::gather_grid(((int64_t)1 << 26) - 1, true, 1);
        expect(bf.xcd_chunk == 32 && bf.blocks * 2 >= ((int64_t)1 << 26) - 1 && bf.blocks * 64 < ((int64_t)1 << 32),
               "bf16 reader grid at the limit", 0);
    }

    expect(spread_runs > 0, "some runs spread their kv workgroups", 0);
    std::printf("cases %lld, valid argument sets %lld, launch shapes %lld, runs launched %lld (kv spread %lld), "
                "gathers launched %lld, mxfp8 launched %lld, contract failures %d\n", cases, ok_validate, ok_shape,
                runs_ok, spread_runs, gathers_ok, mx_ok, failures);
    return failures ? 1 : 0;
}
