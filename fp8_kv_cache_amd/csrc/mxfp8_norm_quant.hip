// Residual add + Gemma RMSNorm + MXFP8 quantization for gfx950 (the second
// operator of include/qkv_prep_mxfp8.h).  A workgroup takes one row, cut into
// K = ceil(hidden / 512) groups of 64 16-byte chunks; each wavefront holds G
// groups (G = 2, or 1 for odd K), lane l holding chunk l of each, so every load
// and store instruction is one coalesced 1 KiB segment.  When hidden is not a
// multiple of 512 the last group is partial (16, 32 or 48 of its 64 chunks);
// its other lanes load nothing, store nothing and add zeros to the sum.
// Each wavefront reduces its groups with the same DPP + permlane order as the
// main operator and leaves the group sums in LDS; after one barrier every
// wavefront adds the K group sums in adjacent pairs, carrying an odd last one,
// so all of them hold the same bits.  That is the numerics contract's order:
// the chunk-level tree with an odd element carried up equals the tree over the
// row padded with zero chunks to whole groups, since x + 0 = x.  A 32-element
// scale block is 4 consecutive chunks held by 4 consecutive lanes, so its amax
// is two DPP max steps; the 4 scale bytes of 4 consecutive blocks (one aligned
// word of the swizzled layout) are gathered into the first lane of each
// 16-lane row and stored as one 4-byte word.
#include "mxfp8_launch.h"
#include "qkvp_device.h"

namespace qkvp {
namespace {

using namespace dev;

__device__ __forceinline__ uint32_t max4(uint32_t v)
{
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    return v;
}

constexpr int kDppRowShl4 = 0x104;   // lane i of a 16-lane row reads lane i + 4 (0 past the row)
constexpr int kDppRowShl8 = 0x108;
constexpr int kDppRowShl12 = 0x10c;

// G groups of 64 chunks per wavefront, K / G wavefronts per row.  PARTIAL:
// some of the K groups' chunks lie past the row (hidden not a multiple of 512,
// or an empty group added to even out K); without it every lane is in range
// and the range checks compile away.
template <int K, int G, bool HAS_RES, bool PARTIAL>
__global__ __launch_bounds__(1024) void mxfp8_kernel(MxArgs a)
{
    static_assert(K % G == 0, "groups must split evenly over the wavefronts");
    __shared__ float group_sum[K];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = blockIdx.x;
    if (row >= a.m) {
        // Padding rows of the last 128-row tile: zero scale bytes, one aligned
        // word of 4 columns per lane.
        for (int c = threadIdx.x * 4; c < a.padded_cols; c += blockDim.x * 4)
            *reinterpret_cast<uint32_t *>(a.scale_out + mx_swizzled_offset(row, c, a.padded_cols)) = 0u;
        return;
    }
    const int64_t rbase = row * a.hidden;
    auto in_row = [&](int chunk) { return !PARTIAL || chunk < a.chunks; };
    u32x4 p[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int chunk = (int)((w * G + j) * 64 + lane);
        p[j] = u32x4{0u, 0u, 0u, 0u};
        if (in_row(chunk)) {
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
    }
    if (a.residual_out) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int chunk = (int)((w * G + j) * 64 + lane);
            if (in_row(chunk))
                store_sys(a.residual_out + rbase, (uint32_t)a.hidden * 2u, (uint32_t)chunk * 16u, p[j]);
        }
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
        if (in_row(chunk))
            unpack_bf16x8(reinterpret_cast<const u32x4 *>(a.gamma)[chunk], gm);
        else
#pragma unroll
            for (int e = 0; e < 8; ++e)
                gm[e] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            nv[e] = (x[e] * inv) * (gm[e] + 1.0f);
        unpack_bf16x8(pack_bf16x8<true>(nv), n);          // rounded to bf16
        uint32_t mx = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            mx = max(mx, __float_as_uint(n[e]) & 0x7fffffffu);
        const float amax = __uint_as_float(max4(mx));
        const uint32_t byte = ue8m0_byte_up(amax * inv448);
        const float inverse = ue8m0_inverse_scale(byte);
        float q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            q[e] = fminf(fmaxf(n[e] * inverse, -448.0f), 448.0f);
        const u32x2 codes = {pack_e4m3<true>(q[0], q[1], q[2], q[3]), pack_e4m3<true>(q[4], q[5], q[6], q[7])};
        // Lane 16r of each 16-lane row holds blocks 4r'..4r'+3 of its group:
        // bytes from itself and lanes +4, +8, +12 (the first lane of each block).
        const uint32_t word = byte | (dpp_u32<kDppRowShl4>(byte) << 8) | (dpp_u32<kDppRowShl8>(byte) << 16) |
                              (dpp_u32<kDppRowShl12>(byte) << 24);
        if (in_row(chunk)) {
            store_sys2(a.quant_out + rbase, (uint32_t)a.hidden, (uint32_t)chunk * 8u, codes);
            if ((lane & 15) == 0)
                *reinterpret_cast<uint32_t *>(a.scale_out + mx_swizzled_offset(row, chunk >> 2, a.padded_cols)) = word;
        }
    }
}

// K groups of 64 chunks per row, mx_groups_per_wave(K) of them per
// wavefront (mxfp8_launch.h has the choice and its measurements).
template <int K>
hipError_t launch_k(const MxArgs &a, hipStream_t st)
{
    if constexpr (!mx_launchable(K)) {
        return hipErrorInvalidValue;
    } else {
        constexpr int G = mx_groups_per_wave(K);
        static_assert(K / G <= 16, "at most 1024 lanes per workgroup");
        const dim3 grid((uint32_t)a.rows_padded), block(64u * (K / G));
        const bool partial = a.chunks != K * 64;
        if (a.residual) {
            if (partial)
                hipLaunchKernelGGL((mxfp8_kernel<K, G, true, true>), grid, block, 0, st, a);
            else
                hipLaunchKernelGGL((mxfp8_kernel<K, G, true, false>), grid, block, 0, st, a);
        } else {
            if (partial)
                hipLaunchKernelGGL((mxfp8_kernel<K, G, false, true>), grid, block, 0, st, a);
            else
                hipLaunchKernelGGL((mxfp8_kernel<K, G, false, false>), grid, block, 0, st, a);
        }
        return hipGetLastError();
    }
}

template <int... Ks>
hipError_t launch_table(const MxArgs &a, hipStream_t st, int k, std::integer_sequence<int, Ks...>)
{
    hipError_t rc = hipErrorInvalidValue;
    (void)((k == Ks + 1 ? (rc = launch_k<Ks + 1>(a, st), true) : false) || ...);
    return rc;
}

}  // namespace

hipError_t launch_mxfp8(const MxArgs &a, hipStream_t st)
{
    return launch_table(a, st, mx_launch_groups(a.hidden), std::make_integer_sequence<int, kMxMaxGroups>{});
}

}  // namespace qkvp
