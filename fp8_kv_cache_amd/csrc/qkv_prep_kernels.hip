// Fused q/kv RMSNorm + RoPE + FP8 (E4M3, UE8M0 block scales) quantize +
// paged KV-cache insert, hand-written for gfx950 (CDNA4, wave64).
//
// What is computed is the per-token operator of the FlagGems-vllm PR 684 page
// (fused_deepseek_v4_qnorm_rope_kv_rope_quant_insert) and its kv half on the
// sglang PR 33358 page (DSv4 flashmla norm-rope-store); the arithmetic is the
// one stated in include/qkv_prep.h.  The operator is HBM bound (about 4 bytes
// of traffic per q element, a handful of fp32 operations), so nothing here is a
// contraction and no MFMA is used.
//
// Work decomposition (a gfx950 design, not the pages' Triton/CUDA tilings):
//  * A wavefront works on a "set" of 4 rows at once, 16 lanes (a DPP row) per
//    512-wide row.  Lane j of a row holds the 16-byte chunks j, j+16, j+32 and
//    j+48 (8 bf16 each), so each load/store instruction moves 4 x 256
//    contiguous bytes, fully coalesced.
//  * The sum of squares follows the fixed order of the numerics contract:
//    each chunk sequentially, then adjacent chunk pairs.  Within a 16-lane row
//    the first four tree levels are DPP adds (quad_perm xor1, xor2,
//    row_half_mirror, row_mirror); levels five and six are in-lane adds of the
//    four chunk groups.  No cross-row permute or LDS is needed.
//  * All heads of a token share one cos/sin row (the Ascend 910B section of the
//    FlagGems page removes a per-head re-gather); here only the 8 lanes that
//    hold rope chunks read it, 32 bytes each.
//  * Several sets' loads are issued before any arithmetic (the sglang page's
//    "K tokens per block" load-level parallelism, as sets per wavefront), and
//    the once-read q/kv rows use non-temporal loads and stores.
//  * q sets and kv sets go to different workgroups of the same launch (the
//    FlagGems page merges the Q and KV launches); kv workgroups come first in
//    dispatch order, so their quantization work overlaps the q stream instead
//    of trailing it.
#include "qkv_prep_internal.h"

namespace qkvp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ memory

__device__ __forceinline__ u32x4 load_stream(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_stream2(u32x2 *p, u32x2 v) { __builtin_nontemporal_store(v, p); }

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_elem(const u32x4 &d, int e)
{
    const uint32_t u = d[e >> 1];
    return (e & 1) ? __uint_as_float(u & 0xffff0000u) : __uint_as_float(u << 16);
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even.
template <bool HW>
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    if constexpr (HW) {
        // fptrunc to bf16 is round-to-nearest-even; gfx950 lowers it to
        // v_cvt_pk_bf16_f32.
        bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
        a = (a + 0x7fffu + ((a >> 16) & 1u)) >> 16;
        b = (b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u;
        return a | b;
    }
}

// ------------------------------------------------------------------ E4M3

// |s| <= 448 by construction (the block scale makes it so).  Integer path:
// round the fp32 significand to 3 bits (ties to even) and rebias the exponent
// from 127 to 7; below 2^-6 the codes are m * 2^-9, m = rint(|s| * 512).
__device__ __forceinline__ uint32_t e4m3_int(float s)
{
    const uint32_t u = __float_as_uint(s);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t code;
    if (a >= 0x3c800000u) {
        const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
        code = min(r - (120u << 3), 0x7eu);
    } else {
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    }
    return code | sign;
}

template <bool HW>
__device__ __forceinline__ uint32_t pack_e4m3(float v0, float v1, float v2, float v3)
{
    if constexpr (HW) {
        // v_cvt_pk_fp8_f32: two values into one 16-bit half, OCP e4m3,
        // round to nearest even.
        uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
        return __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, r, true);
    } else {
        return e4m3_int(v0) | (e4m3_int(v1) << 8) | (e4m3_int(v2) << 16) | (e4m3_int(v3) << 24);
    }
}

// Least e with amax <= 448 * 2^e, clamped to [-127, 127]; amax given as the
// bits of a non-negative finite float.  448 = 1.75 * 2^8, so for a normal
// amax = (1 + f) 2^E the answer is E - 8, plus one when f > 0.75.  A zero or
// subnormal amax is below 448 * 2^-127 and clamps to -127.
__device__ __forceinline__ int ue8m0_exponent(uint32_t amax_bits)
{
    const uint32_t ef = amax_bits >> 23;
    if (ef == 0)
        return -127;
    const int e = (int)ef - 135 + ((amax_bits & 0x7fffffu) > 0x600000u ? 1 : 0);
    return e < -127 ? -127 : e;
}

// ------------------------------------------------------------------ DPP

constexpr int quad_perm(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }
constexpr int kDppXor1 = quad_perm(1, 0, 3, 2);
constexpr int kDppXor2 = quad_perm(2, 3, 0, 1);
constexpr int kDppHalfMirror = 0x141;  // lane i of an 8-lane half reads lane 7-i
constexpr int kDppMirror = 0x140;      // lane i of a 16-lane row reads lane 15-i
constexpr int kDppRor8 = 0x128;        // lane i of a 16-lane row reads lane (i+8) mod 16

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

// Tree levels 1-4 over the 16 lanes of a DPP row.  After each level both
// partners hold the same bits (IEEE addition commutes), so mirrors act as
// xor-4 and xor-8 exchanges.
__device__ __forceinline__ float tree16(float v)
{
    v = v + dpp_f32<kDppXor1>(v);
    v = v + dpp_f32<kDppXor2>(v);
    v = v + dpp_f32<kDppHalfMirror>(v);
    v = v + dpp_f32<kDppMirror>(v);
    return v;
}

// Max over the 8-lane half of a DPP row (one quantization block of 64 dims).
__device__ __forceinline__ uint32_t max8(uint32_t v)
{
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    return v;
}

// ------------------------------------------------------------------ row math

__device__ __forceinline__ float chunk_sum_squares(const u32x4 &d)
{
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = bf16_elem(d, e);
        acc = __builtin_fmaf(x, x, acc);  // x*x is exact for bf16 x
    }
    return acc;
}

// inv = 1 / sqrt(S/512 + eps): S * 2^-9 is the correctly rounded S/512;
// __builtin_sqrtf and '/' are the correctly rounded IEEE operations.
__device__ __forceinline__ float inv_rms(const u32x4 (&d)[4], float eps)
{
    const float g0 = tree16(chunk_sum_squares(d[0]));
    const float g1 = tree16(chunk_sum_squares(d[1]));
    const float g2 = tree16(chunk_sum_squares(d[2]));
    const float g3 = tree16(chunk_sum_squares(d[3]));
    const float s = (g0 + g1) + (g2 + g3);
    const float v = s * 0.001953125f + eps;
    return 1.0f / __builtin_sqrtf(v);
}

template <bool HAS_W>
__device__ __forceinline__ void normalize8(const u32x4 &x, const u32x4 &w, float inv, float (&y)[8])
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float t = bf16_elem(x, e) * inv;
        y[e] = HAS_W ? t * bf16_elem(w, e) : t;
    }
}

// Rotate the 4 interleaved pairs of one rope chunk.
__device__ __forceinline__ void rope8(float (&y)[8], const f32x4 &c, const f32x4 &s)
{
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float a = y[2 * p], b = y[2 * p + 1];
        const float bs = b * s[p];
        const float bc = b * c[p];
        y[2 * p] = __builtin_fmaf(a, c[p], -bs);
        y[2 * p + 1] = __builtin_fmaf(a, s[p], bc);
    }
}

template <bool HW>
__device__ __forceinline__ u32x4 pack_bf16x8(const float (&y)[8])
{
    return u32x4{pack_bf16<HW>(y[0], y[1]), pack_bf16<HW>(y[2], y[3]),
                 pack_bf16<HW>(y[4], y[5]), pack_bf16<HW>(y[6], y[7])};
}

__device__ __forceinline__ int64_t clamp_position(int64_t p, int64_t max_position)
{
    return p < 0 ? 0 : (p >= max_position ? max_position - 1 : p);
}

// ------------------------------------------------------------------ q sets

// U consecutive sets of 4 q rows.  Every lane takes part in the DPP trees, so
// rows past the end are computed on zeros and simply not stored.
template <int U, bool HAS_W, bool HW>
__device__ __forceinline__ void q_sets(const KernelArgs &a, int64_t set0, uint32_t quarter, uint32_t j)
{
    int64_t row[U];
    bool ok[U];
    int64_t pos[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        row[u] = (set0 + u) * kRowsPerSet + quarter;
        ok[u] = row[u] < a.q_rows;
        const uint32_t tok = ok[u] ? (uint32_t)row[u] / a.num_heads : 0u;
        pos[u] = a.positions[tok];
    }
    u32x4 d[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(a.q + row[u] * kHeadDim) + j;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            d[u][k] = ok[u] ? load_stream(src + 16 * k) : u32x4{0u, 0u, 0u, 0u};
    }
    u32x4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = HAS_W ? reinterpret_cast<const u32x4 *>(a.q_w)[j + 16 * k] : u32x4{0u, 0u, 0u, 0u};
    f32x4 cv[U], sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        cv[u] = f32x4{1.f, 1.f, 1.f, 1.f};
        sv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j >= 8) {
            const f32x4 *cs = reinterpret_cast<const f32x4 *>(
                a.cos_sin + clamp_position(pos[u], a.max_position) * kRopeDim);
            cv[u] = cs[j - 8];
            sv[u] = cs[j];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float inv = inv_rms(d[u], a.eps);
        u32x4 *dst = reinterpret_cast<u32x4 *>(a.q + row[u] * kHeadDim) + j;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float y[8];
            normalize8<HAS_W>(d[u][k], w[k], inv, y);
            if (k == 3 && j >= 8)
                rope8(y, cv[u], sv[u]);
            const u32x4 out = pack_bf16x8<HW>(y);
            if (ok[u])
                store_stream(dst + 16 * k, out);
        }
    }
}

// ------------------------------------------------------------------ kv sets

// One set = the kv rows of 4 consecutive tokens, one per 16-lane row.  In lane
// j, chunk register k holds dims 8(j+16k)..+7, i.e. quantization block
// 2k + (j >= 8); register 3 of lanes 8..15 is the rope chunk.
template <bool HW>
__device__ __forceinline__ void kv_set(const KernelArgs &a, int64_t set, uint32_t quarter, uint32_t j)
{
    const int64_t t = set * kRowsPerSet + quarter;
    const int64_t slot = t < a.num_tokens ? a.slot_mapping[t] : -1;
    const bool valid = slot >= 0 && slot < a.num_slots;
    const int64_t pos = valid ? a.positions[t] : 0;
    u32x4 d[4], w[4];
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.kv + t * kHeadDim) + j;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        d[k] = valid ? load_stream(src + 16 * k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = reinterpret_cast<const u32x4 *>(a.kv_w)[j + 16 * k];
    f32x4 cv = f32x4{1.f, 1.f, 1.f, 1.f}, sv = f32x4{0.f, 0.f, 0.f, 0.f};
    if (j >= 8 && valid) {
        const f32x4 *cs = reinterpret_cast<const f32x4 *>(
            a.cos_sin + clamp_position(pos, a.max_position) * kRopeDim);
        cv = cs[j - 8];
        sv = cs[j];
    }

    const float inv = inv_rms(d, a.eps);
    float y[4][8];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        normalize8<true>(d[k], w[k], inv, y[k]);

    // Block amax over the 8 lanes of a half row, then the UE8M0 exponent.
    uint32_t ebyte[4];
    float inv_scale[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            m = max(m, __float_as_uint(y[k][e]) & 0x7fffffffu);
        const int ex = ue8m0_exponent(max8(m));
        ebyte[k] = (uint32_t)(ex + 127);
        inv_scale[k] = __uint_as_float((uint32_t)(127 - ex) << 23);  // exactly 2^-ex
    }
    uint32_t epart[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        epart[k] = dpp_u32<kDppRor8>(ebyte[k]);  // the other half row's block

    if (j >= 8)
        rope8(y[3], cv, sv);

    if (!valid)
        return;
    const uint32_t s32 = (uint32_t)slot;
    const uint32_t blk = s32 / a.block_size;
    const uint32_t sib = s32 - blk * a.block_size;
    uint8_t *base = a.cache + (int64_t)blk * a.block_size * kSlotBytes;
    uint8_t *data = base + (int64_t)sib * kSlotData;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (k < 3 || j < 8) {
            const float sc = inv_scale[k];
            const u32x2 codes = {
                pack_e4m3<HW>(y[k][0] * sc, y[k][1] * sc, y[k][2] * sc, y[k][3] * sc),
                pack_e4m3<HW>(y[k][4] * sc, y[k][5] * sc, y[k][6] * sc, y[k][7] * sc)};
            store_stream2(reinterpret_cast<u32x2 *>(data) + (j + 16 * k), codes);
        } else {
            store_stream(reinterpret_cast<u32x4 *>(data + kNopeDim) + (j - 8), pack_bf16x8<HW>(y[3]));
        }
    }
    if (j == 0) {
        // Blocks 0, 2, 4, 6 are this lane's; 1, 3, 5 come from lane 8.
        const u32x2 rec = {ebyte[0] | (epart[0] << 8) | (ebyte[1] << 16) | (epart[1] << 24),
                           ebyte[2] | (epart[2] << 8) | (ebyte[3] << 16)};
        store_stream2(reinterpret_cast<u32x2 *>(base + (int64_t)a.block_size * kSlotData +
                                                (int64_t)sib * kSlotScale),
                      rec);
    }
}

// ------------------------------------------------------------------ kernel

template <int U, bool HAS_W, bool HW>
__global__ __launch_bounds__(512) void qkv_prep_kernel(KernelArgs a)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t quarter = lane >> 4;
    const uint32_t j = lane & 15u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t waves_per_block = blockDim.x >> 6;
    if (blockIdx.x < a.kv_blocks) {
        const int64_t set = (int64_t)blockIdx.x * waves_per_block + wave;
        if (set < a.kv_sets)
            kv_set<HW>(a, set, quarter, j);
    } else {
        const int64_t wv = (int64_t)(blockIdx.x - a.kv_blocks) * waves_per_block + wave;
        const int64_t set0 = wv * U;
        if (set0 < a.q_sets)
            q_sets<U, HAS_W, HW>(a, set0, quarter, j);
    }
}

template <int U, bool HAS_W, bool HW>
hipError_t launch_variant(const KernelArgs &a, dim3 grid, dim3 block, hipStream_t stream)
{
    hipLaunchKernelGGL((qkv_prep_kernel<U, HAS_W, HW>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <int U>
hipError_t launch_u(const KernelArgs &a, bool has_w, bool hw, dim3 grid, dim3 block, hipStream_t st)
{
    if (has_w)
        return hw ? launch_variant<U, true, true>(a, grid, block, st)
                  : launch_variant<U, true, false>(a, grid, block, st);
    return hw ? launch_variant<U, false, true>(a, grid, block, st)
              : launch_variant<U, false, false>(a, grid, block, st);
}

}  // namespace

hipError_t launch_qkv_prep(const KernelArgs &a, const LaunchShape &s, hipStream_t stream)
{
    const dim3 grid((uint32_t)(s.kv_blocks + s.q_blocks));
    const dim3 block(64u * (uint32_t)s.waves_per_block);
    const bool has_w = a.q_w != nullptr;
    const bool hw = s.convert == 2;
    switch (s.sets_per_wave) {
    case 1: return launch_u<1>(a, has_w, hw, grid, block, stream);
    case 2: return launch_u<2>(a, has_w, hw, grid, block, stream);
    case 4: return launch_u<4>(a, has_w, hw, grid, block, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qkvp
