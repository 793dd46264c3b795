// Host-only fuzz of the C ABI's argument checks and launch heuristic, built
// with -fsanitize=address,undefined by tests/test_host_sanitized.py and linked
// against the host API with the two kernel launchers stubbed out (nothing here
// touches a GPU).  Extreme and random configs and arguments go through
// qkv_prep_validate, qkv_prep_launch_shape, qkv_prep_supported and
// qkv_prep_strerror; any undefined operation aborts the run, and the returned
// values are checked against the documented contract.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "qkv_prep.h"
#include "qkv_prep_gather.h"
#include "qkv_prep_launch.h"

namespace qkvp {
hipError_t launch_qkv_prep(const KernelArgs &, const LaunchShape &, hipStream_t) { return hipSuccess; }
hipError_t launch_gather(const GatherArgs &, int, hipStream_t) { return hipSuccess; }
}  // namespace qkvp

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

        const int64_t T = next() % 2 ? (int64_t)(next() % 200000) : pick64();
        qkv_prep_launch sh;
        const int rs = qkv_prep_launch_shape(&c, (int32_t)(next() % 512), T, &sh);
        expect(rs >= 0 && rs <= 6, "launch_shape code", i);
        if (rs == QKV_PREP_OK) {
            ++ok_shape;
            expect(sh.grid == sh.kv_blocks + sh.q_blocks, "grid = kv + q", i);
            expect(sh.kv_blocks >= 0 && sh.q_blocks >= 0, "non-negative blocks", i);
            expect(sh.rows_per_wave == 1 || sh.rows_per_wave == 2 || sh.rows_per_wave == 4, "rows per wave", i);
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
            expect((sh.kv_blocks + sh.q_blocks) * 64 * sh.waves_per_block < ((int64_t)1 << 32),
                   "dispatch fits 32-bit work-item count", i);
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
    std::printf("cases %lld, valid argument sets %lld, launch shapes %lld, contract failures %d\n", cases,
                ok_validate, ok_shape, failures);
    return failures ? 1 : 0;
}
