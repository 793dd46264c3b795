// Device helpers shared by the gfx950 kernels of this library: vector types,
// streaming loads/stores, fixed-point division, bf16 and E4M3 packing, the
// UE8M0 exponent of the main operator, and the ordered 64-lane sum.
#pragma once

#include "qkv_prep_internal.h"

namespace qkvp {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ memory

__device__ __forceinline__ u32x4 load_stream(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_stream2(u32x2 *p, u32x2 v) { __builtin_nontemporal_store(v, p); }

// Stores with the non-temporal, system-scope cache policy (the nt and sc1
// bits), issued through a buffer descriptor: a global store cannot carry sc1
// from source.  Measured on MI355X with 2 GiB buffers, this store policy lifts
// a streaming copy from ~6.46 to ~6.70 TB/s and an in-place update from ~6.72
// to ~6.82 TB/s; the load policy makes no difference there.  `base` must be
// wave-uniform (the descriptor lives in scalar registers); a store at or past
// `bytes` from `base` is dropped by the descriptor's range check.
constexpr int kPolicyNtSc1 = 2 | 16;             // nt | sc1
constexpr int kRawBufferWord3 = 0x00020000;      // 32-bit data format, no swizzle (gfx9)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, kRawBufferWord3);
}

__device__ __forceinline__ void store_sys(void *base, uint32_t bytes, uint32_t off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, stream_rsrc(base, bytes), (int)off, 0, kPolicyNtSc1);
}

__device__ __forceinline__ void store_sys2(void *base, uint32_t bytes, uint32_t off, u32x2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, stream_rsrc(base, bytes), (int)off, 0, kPolicyNtSc1);
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, FastDiv d)
{
    return (__umulhi(n, d.mul) + n) >> d.shift;
}

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ void unpack_bf16x8(const u32x4 &d, float (&x)[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(d[i] << 16);
        x[2 * i + 1] = __uint_as_float(d[i] & 0xffff0000u);
    }
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

template <bool HW>
__device__ __forceinline__ u32x4 pack_bf16x8(const float (&y)[8])
{
    return u32x4{pack_bf16<HW>(y[0], y[1]), pack_bf16<HW>(y[2], y[3]),
                 pack_bf16<HW>(y[4], y[5]), pack_bf16<HW>(y[6], y[7])};
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

// The MXFP8 scale byte of v: the least b >= 0 with v <= 2^(b - 127), at most
// 254; 0 for v <= 0 (v finite).  Positive floats order like their bit
// patterns, and 2^(b - 127) has the pattern b << 23 for b >= 1, so the least
// b >= 1 is the pattern divided by 2^23, rounded up.  Patterns up to
// 0x00400000 (2^-127, a subnormal) give b = 0; as a signed integer, every
// negative value and -0 fall in that case too.
__device__ __forceinline__ uint32_t ue8m0_byte_up(float v)
{
    const uint32_t u = __float_as_uint(v);
    if ((int32_t)u <= 0x00400000)
        return 0u;
    return min((u + 0x7fffffu) >> 23, 254u);
}

// The inverse of a scale byte: 2^(127 - byte) for bytes 1..253; 0 for byte 0
// (a zero block) and for 254, whose power 2^-127 is below the normal range.
__device__ __forceinline__ float ue8m0_inverse_scale(uint32_t byte)
{
    return byte - 1u < 253u ? __builtin_ldexpf(1.0f, 127 - (int)byte) : 0.0f;
}

// ------------------------------------------------------------------ cross-lane

constexpr int quad_perm(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }
constexpr int kDppXor1 = quad_perm(1, 0, 3, 2);
constexpr int kDppXor2 = quad_perm(2, 3, 0, 1);
constexpr int kDppHalfMirror = 0x141;  // lane i of an 8-lane half reads lane 7-i
constexpr int kDppMirror = 0x140;      // lane i of a 16-lane row reads lane 15-i

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

// Sum over all 64 lanes in the adjacent-pairs order.  Levels 1-4 inside each
// 16-lane row: after each level both partners hold the same bits (IEEE
// addition commutes), so the mirrors act as xor-4 and xor-8 exchanges.
// Level 5: v_permlane16_swap(v, v) yields rows (0,0,2,2) and (1,1,3,3), whose
// sum is row0+row1 | row2+row3 in every lane.  Level 6: v_permlane32_swap(s, s)
// yields halves (lo, lo) and (hi, hi).
__device__ __forceinline__ float wave_sum_ordered(float v)
{
    v = v + dpp_f32<kDppXor1>(v);
    v = v + dpp_f32<kDppXor2>(v);
    v = v + dpp_f32<kDppHalfMirror>(v);
    v = v + dpp_f32<kDppMirror>(v);
    const uint32_t b = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    const float s = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const uint32_t c = __float_as_uint(s);
    const auto h = __builtin_amdgcn_permlane32_swap(c, c, false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

// Max over the 8-lane half of a DPP row (one quantization block of 64 dims).
__device__ __forceinline__ uint32_t max8(uint32_t v)
{
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    return v;
}

}  // namespace dev
}  // namespace qkvp
