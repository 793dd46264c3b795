// Residual add + Gemma RMSNorm + MXFP8 quantization for gfx950 (the second
// operator of include/qkv_prep_mxfp8.h).  A workgroup takes one row of
// K = hidden / 512 groups of 64 16-byte chunks; each wavefront holds G groups
// (G = 2, or 1 for odd K), lane l holding chunk l of each, so every load and
// store instruction is one coalesced 1 KiB segment.  Each wavefront reduces
// its groups with the same DPP + permlane order as the main operator and
// leaves the group sums in LDS; after one barrier every wavefront adds the K
// group sums in adjacent pairs, carrying an odd last one (the numerics
// contract's order), so all of them hold the same bits.  A 32-element scale
// block is 4 consecutive chunks held by 4 consecutive lanes, so its amax is
// two DPP max steps.
#include "mxfp8_launch.h"
#include "qkvp_device.h"

namespace qkvp {
namespace {

using namespace dev;

__device__ __forceinline__ int64_t swizzled_offset(int64_t row, int64_t col, int64_t padded_cols)
{
    return (col & 3) + (col >> 2) * 512 + (row & 31) * 16 + ((row & 127) >> 5) * 4 + (row >> 7) * 128 * padded_cols;
}

// The page's rounded-up biased exponent of v.
__device__ __forceinline__ uint32_t ue8m0_ceil_byte(float v)
{
    if (!(v > 0.0f))
        return 0;
    const uint32_t bits = __float_as_uint(v);
    const uint32_t e = bits >> 23;
    const uint32_t mant = bits & 0x7fffffu;
    const uint32_t bump = (mant != 0 && !(e == 0 && mant <= 0x400000u)) ? 1u : 0u;
    return min(e + bump, 254u);
}

__device__ __forceinline__ uint32_t max4(uint32_t v)
{
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    return v;
}

// G groups of 64 chunks per wavefront, K / G wavefronts per row.
template <int K, int G, bool HAS_RES>
__global__ __launch_bounds__(1024) void mxfp8_kernel(MxArgs a)
{
    static_assert(K % G == 0, "groups must split evenly over the wavefronts");
    __shared__ float group_sum[K];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = blockIdx.x;
    if (row >= a.m) {
        // Padding rows of the last 128-row tile: zero scale bytes.
        for (int c = threadIdx.x; c < a.padded_cols; c += blockDim.x)
            a.scale_out[swizzled_offset(row, c, a.padded_cols)] = 0;
        return;
    }
    const int64_t rbase = row * a.hidden;
    u32x4 p[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int chunk = (int)((w * G + j) * 64 + lane);
        const u32x4 xv = load_stream(reinterpret_cast<const u32x4 *>(a.x + rbase) + chunk);
        if constexpr (HAS_RES) {
            const u32x4 rv = load_stream(reinterpret_cast<const u32x4 *>(a.residual + rbase) + chunk);
            float xf[8], rf[8], sf[8];
            unpack_bf16x8(xv, xf);
            unpack_bf16x8(rv, rf);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sf[e] = xf[e] + rf[e];
            p[j] = pack_bf16x8<true>(sf);
        } else {
            p[j] = xv;
        }
    }
    if (a.residual_out) {
#pragma unroll
        for (int j = 0; j < G; ++j)
            store_sys(a.residual_out + rbase, (uint32_t)a.hidden * 2u, ((w * G + j) * 64 + lane) * 16u, p[j]);
    }
    float g[K];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        float x[8];
        unpack_bf16x8(p[j], x);
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc = __builtin_fmaf(x[e], x[e], acc);
        g[j] = wave_sum_ordered(acc);
    }
    if constexpr (K != G) {
        // Several wavefronts per row: exchange the group sums through LDS.
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < G; ++j)
                group_sum[w * G + j] = g[j];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < K; ++j)
            g[j] = group_sum[j];
    }
#pragma unroll
    for (int n = K; n > 1; n = (n + 1) / 2) {
#pragma unroll
        for (int i = 0; i < n / 2; ++i)
            g[i] = g[2 * i] + g[2 * i + 1];
        if (n % 2)
            g[n / 2] = g[n - 1];
    }
    const float inv = 1.0f / __builtin_sqrtf(g[0] / (float)a.hidden + a.eps);
    const float inv448 = 1.0f / 448.0f;

#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int chunk = (int)((w * G + j) * 64 + lane);
        float x[8], gm[8], nv[8], n[8];
        unpack_bf16x8(p[j], x);
        unpack_bf16x8(reinterpret_cast<const u32x4 *>(a.gamma)[chunk], gm);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            nv[e] = (x[e] * inv) * (gm[e] + 1.0f);
        unpack_bf16x8(pack_bf16x8<true>(nv), n);          // rounded to bf16
        uint32_t mx = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            mx = max(mx, __float_as_uint(n[e]) & 0x7fffffffu);
        const float amax = __uint_as_float(max4(mx));
        const uint32_t byte = ue8m0_ceil_byte(amax * inv448);
        const int32_t ne = 254 - (int32_t)byte;
        const float inverse = byte == 0 ? 0.0f : __uint_as_float((uint32_t)(ne > 0 ? ne : 0) << 23);
        float q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            q[e] = fminf(fmaxf(n[e] * inverse, -448.0f), 448.0f);
        const u32x2 codes = {pack_e4m3<true>(q[0], q[1], q[2], q[3]), pack_e4m3<true>(q[4], q[5], q[6], q[7])};
        store_sys2(a.quant_out + rbase, (uint32_t)a.hidden, (uint32_t)chunk * 8u, codes);
        if ((lane & 3) == 0)
            a.scale_out[swizzled_offset(row, chunk >> 2, a.padded_cols)] = (uint8_t)byte;
    }
}

// Groups of 64 chunks per wavefront for a row of K groups.  Measured on
// MI355X at hidden 1024-8192 (two interleaved rounds): two groups per
// wavefront (K/2 wavefronts per row) is the fastest or tied everywhere; one
// group per wavefront is within 2%; one wavefront per row loses up to 60% at
// large K (VGPR pressure).  Odd K uses one group per wavefront.
constexpr int groups_per_wave(int K) { return K % 2 == 0 ? 2 : 1; }

template <int K>
hipError_t launch_k(const MxArgs &a, hipStream_t st)
{
    constexpr int G = groups_per_wave(K);
    const dim3 grid((uint32_t)a.rows_padded), block(64u * (K / G));
    if (a.residual)
        hipLaunchKernelGGL((mxfp8_kernel<K, G, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((mxfp8_kernel<K, G, false>), grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mxfp8(const MxArgs &a, hipStream_t st)
{
    switch (a.hidden / 512) {
    case 1: return launch_k<1>(a, st);
    case 2: return launch_k<2>(a, st);
    case 3: return launch_k<3>(a, st);
    case 4: return launch_k<4>(a, st);
    case 5: return launch_k<5>(a, st);
    case 6: return launch_k<6>(a, st);
    case 7: return launch_k<7>(a, st);
    case 8: return launch_k<8>(a, st);
    case 9: return launch_k<9>(a, st);
    case 10: return launch_k<10>(a, st);
    case 11: return launch_k<11>(a, st);
    case 12: return launch_k<12>(a, st);
    case 13: return launch_k<13>(a, st);
    case 14: return launch_k<14>(a, st);
    case 15: return launch_k<15>(a, st);
    case 16: return launch_k<16>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qkvp
