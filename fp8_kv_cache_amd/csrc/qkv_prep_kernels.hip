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
//  * One wavefront per 512-wide row: lane l holds the 16-byte chunk l (dims
//    8l..8l+7), so a row is one fully coalesced 1 KiB load and one 1 KiB store.
//    Measured on MI355X, this shape streams at the copy ceiling at every
//    footprint (~6.5 TB/s with non-temporal stores), while shapes with several
//    loads per lane in flight (4 rows per wave, or several rows per wave) lose
//    6-15% once the footprint passes a few GiB.  Workgroups of one wavefront,
//    or two where the launch heuristic pairs the two-heads shape with several
//    kv tokens per wavefront; non-temporal loads.
//  * Stores: with one row per wavefront every store carries the non-temporal
//    system-scope policy (nt sc1), 1-2.5% faster than plain non-temporal
//    stores from 32768x64 up (about 2% at 32768x128 and 131072x128).  The
//    two-heads shape keeps plain non-temporal stores: with nt sc1 it was
//    3-18% slower on small batches (footprints within the MALL) and within
//    noise on large few-head ones.
//  * The sum of squares follows the fixed order of the numerics contract: each
//    chunk sequentially, then adjacent chunk pairs.  Levels 1-4 are DPP adds
//    inside a 16-lane row (quad_perm xor1, xor2, row_half_mirror, row_mirror);
//    level 5 pairs rows 0+1 and 2+3 with v_permlane16_swap and level 6 pairs
//    the halves with v_permlane32_swap (both gfx950 instructions).  Every lane
//    ends with the same bits.  No LDS.
//  * A wavefront's row belongs to one token, so the token index (a fixed-point
//    division by H), the position and the cos/sin row address are wave-uniform
//    scalar values; only the 8 lanes holding rope chunks read the table
//    (all heads of a token share it: the Ascend 910B section of the FlagGems
//    page removes a per-head re-gather).
//  * q rows and kv rows go to different workgroups of one launch (the FlagGems
//    page merges the Q and KV launches); kv workgroups come first in dispatch
//    order, so their quantization overlaps the q stream instead of trailing it
//    (for large two-heads batches they are spread over the first 55-75% of
//    the grid instead; the launch heuristic says when).
//    Where the launch heuristic says so, a kv wavefront takes two or four
//    consecutive tokens, all their loads issued together: the kv wavefronts
//    form a latency-bound burst at the start, and more loads in flight per
//    wavefront shorten it.
//  * Depending on the token and head counts, a wavefront takes two heads of
//    one token, one after the other, so the token's position, cos/sin row and
//    the q weight are loaded once per two rows (the launch heuristic in
//    qkv_prep_api.cpp says when, with its measurements).
//    Issuing several q rows' loads at once (the sglang page's "K tokens per
//    block" load-level parallelism) was slower at every size measured; the kv
//    burst above is the one place where it pays.
#include "qkv_prep_launch.h"
#include "qkvp_device.h"

namespace qkvp {
namespace {

using namespace dev;

constexpr int kRopeLane = kNopeDim / 8;  // lanes 56..63 hold the rope chunks
constexpr int kBf16SlotBytes = 1024;

// ------------------------------------------------------------------ row math

// inv = 1 / sqrt(S/512 + eps).  S * 2^-9 is the correctly rounded S/512;
// __builtin_sqrtf and '/' are the correctly rounded IEEE operations.
__device__ __forceinline__ float inv_rms(const float (&x)[8], float eps)
{
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc = __builtin_fmaf(x[e], x[e], acc);  // x*x is exact for bf16 x
    const float s = wave_sum_ordered(acc);
    const float v = s * 0.001953125f + eps;
    return 1.0f / __builtin_sqrtf(v);
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

__device__ __forceinline__ int64_t clamp_position(int64_t p, int64_t max_position)
{
    return p < 0 ? 0 : (p >= max_position ? max_position - 1 : p);
}

// ------------------------------------------------------------------ q rows

// One q row per wavefront.  `row` is wave-uniform, so every branch below is
// uniform too, except the rope lanes.
template <bool HAS_W, bool HW>
__device__ __forceinline__ void q_row(const KernelArgs &a, int64_t row, uint32_t lane)
{
    const int64_t pos = a.positions[fastdiv((uint32_t)row, a.heads)];
    const u32x4 d = load_stream(reinterpret_cast<const u32x4 *>(a.q + row * kHeadDim) + lane);
    float w[8];
    if (HAS_W)
        unpack_bf16x8(reinterpret_cast<const u32x4 *>(a.q_w)[lane], w);
    f32x4 cv = f32x4{1.f, 1.f, 1.f, 1.f}, sv = f32x4{0.f, 0.f, 0.f, 0.f};
    if (lane >= kRopeLane) {
        const f32x4 *cs = reinterpret_cast<const f32x4 *>(
            a.cos_sin + clamp_position(pos, a.max_position) * kRopeDim);
        cv = cs[lane - kRopeLane];
        sv = cs[lane - kRopeLane + 8];
    }
    float x[8], y[8];
    unpack_bf16x8(d, x);
    // From the arrival of its row until its store is issued, the wavefront
    // issues ahead of the SIMD's wavefronts still waiting for their loads, so
    // rows leave the chip sooner.  Measured on MI355X (six interleaved rounds,
    // one process): 32768x64 648.8 -> 645.9 us, 131072x128 5167 -> 5146 us,
    // 2048x64 41.52 -> 41.40 us; priority 2 or 3 measure the same, raising it
    // before the loads instead is 6% slower, and doing the same in the kv and
    // two-heads paths gains nothing more.
    __builtin_amdgcn_s_setprio(1);
    const float inv = inv_rms(x, a.eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float t = x[e] * inv;
        y[e] = HAS_W ? t * w[e] : t;
    }
    if (lane >= kRopeLane)
        rope8(y, cv, sv);
    store_sys(a.q + row * kHeadDim, kHeadDim * 2u, lane * 16u, pack_bf16x8<HW>(y));
    __builtin_amdgcn_s_setprio(0);
}

// Heads h0 .. h0+n-1 of one token (n = min(U, H - h0)) on one wavefront, one
// row after another: the token's position, its cos/sin row and the q weight
// are loaded once for the chunk, then each row is loaded, normalized, rotated
// and stored in turn (one row's load in flight, as with one row per
// wavefront).
template <int U, bool HAS_W, bool HW>
__device__ __forceinline__ void q_chunk(const KernelArgs &a, uint32_t wv, uint32_t lane)
{
    const uint32_t t = fastdiv(wv, a.chunk_div);
    const uint32_t h0 = (wv - t * a.chunks) * U;
    const uint32_t n = min((uint32_t)U, a.num_heads - h0);
    const int64_t row0 = (int64_t)t * a.num_heads + h0;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.q + row0 * kHeadDim) + lane;
    u32x4 *dst = reinterpret_cast<u32x4 *>(a.q + row0 * kHeadDim) + lane;
    u32x4 d = load_stream(src);
    float w[8];
    if (HAS_W)
        unpack_bf16x8(reinterpret_cast<const u32x4 *>(a.q_w)[lane], w);
    const int64_t pos = a.positions[t];
    f32x4 cv = f32x4{1.f, 1.f, 1.f, 1.f}, sv = f32x4{0.f, 0.f, 0.f, 0.f};
    if (lane >= kRopeLane) {
        const f32x4 *cs = reinterpret_cast<const f32x4 *>(
            a.cos_sin + clamp_position(pos, a.max_position) * kRopeDim);
        cv = cs[lane - kRopeLane];
        sv = cs[lane - kRopeLane + 8];
    }
    for (uint32_t j = 0; j < n; ++j) {
        float x[8], y[8];
        unpack_bf16x8(d, x);
        const float inv = inv_rms(x, a.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float tt = x[e] * inv;
            y[e] = HAS_W ? tt * w[e] : tt;
        }
        if (lane >= kRopeLane)
            rope8(y, cv, sv);
        store_stream(dst + j * 64, pack_bf16x8<HW>(y));
        if (j + 1 < n)
            d = load_stream(src + (j + 1) * 64);
    }
}

// ------------------------------------------------------------------ kv rows

// One token's kv row, once its slot (valid) and its row `d` are loaded.  Lane
// l < 56 holds dims 8l..8l+7 of quantization block l/8 and writes their 8
// codes; lanes 56..63 hold the rope dims and write 16 bytes of rotated bf16
// each; one lane writes the 8-byte scale record.  SYS: the stores take the nt
// sc1 policy (with the one-row-per-wavefront q path).
template <bool HW, bool SYS>
__device__ __forceinline__ void kv_finish(const KernelArgs &a, int64_t t, int64_t slot, const u32x4 &d,
                                          const float (&w)[8], uint32_t lane)
{
    f32x4 cv = f32x4{1.f, 1.f, 1.f, 1.f}, sv = f32x4{0.f, 0.f, 0.f, 0.f};
    if (lane >= kRopeLane) {
        const f32x4 *cs = reinterpret_cast<const f32x4 *>(
            a.cos_sin + clamp_position(a.positions[t], a.max_position) * kRopeDim);
        cv = cs[lane - kRopeLane];
        sv = cs[lane - kRopeLane + 8];
    }

    float x[8], y[8];
    unpack_bf16x8(d, x);
    const float inv = inv_rms(x, a.eps);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        y[e] = (x[e] * inv) * w[e];

    if (a.bf16_store) {
        // bf16 slot: the rotated row as bf16, slot s at byte s * 1024.
        if (lane >= kRopeLane)
            rope8(y, cv, sv);
        if constexpr (SYS)
            store_sys(a.cache + slot * kBf16SlotBytes, kBf16SlotBytes, lane * 16u, pack_bf16x8<HW>(y));
        else
            store_stream(reinterpret_cast<u32x4 *>(a.cache + slot * kBf16SlotBytes) + lane, pack_bf16x8<HW>(y));
        return;
    }

    // Block amax over the 8 lanes of a half row, then the UE8M0 exponent.
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        m = max(m, __float_as_uint(y[e]) & 0x7fffffffu);
    const int ex = ue8m0_exponent(max8(m));
    const float inv_scale = __uint_as_float((uint32_t)(127 - ex) << 23);  // exactly 2^-ex
    const uint32_t ebyte = (uint32_t)(ex + 127);
    // Exponent bytes of blocks 0..6 (lanes 0, 8, ..., 48), wave-uniform.
    const uint32_t rec0 = __builtin_amdgcn_readlane(ebyte, 0) | (__builtin_amdgcn_readlane(ebyte, 8) << 8) |
                          (__builtin_amdgcn_readlane(ebyte, 16) << 16) |
                          (__builtin_amdgcn_readlane(ebyte, 24) << 24);
    const uint32_t rec1 = __builtin_amdgcn_readlane(ebyte, 32) | (__builtin_amdgcn_readlane(ebyte, 40) << 8) |
                          (__builtin_amdgcn_readlane(ebyte, 48) << 16);

    const uint32_t s32 = (uint32_t)slot;
    const uint32_t blk = fastdiv(s32, a.blocks);
    const uint32_t sib = s32 - blk * a.block_size;
    uint8_t *base = a.cache + (int64_t)blk * a.block_size * kSlotBytes;
    uint8_t *data = base + (int64_t)sib * kSlotData;
    if (lane < kRopeLane) {
        const u32x2 codes = {pack_e4m3<HW>(y[0] * inv_scale, y[1] * inv_scale, y[2] * inv_scale, y[3] * inv_scale),
                             pack_e4m3<HW>(y[4] * inv_scale, y[5] * inv_scale, y[6] * inv_scale, y[7] * inv_scale)};
        if constexpr (SYS)
            store_sys2(data, kSlotData, lane * 8u, codes);
        else
            store_stream2(reinterpret_cast<u32x2 *>(data) + lane, codes);
    } else {
        rope8(y, cv, sv);
        if constexpr (SYS)
            store_sys(data, kSlotData, kNopeDim + (lane - kRopeLane) * 16u, pack_bf16x8<HW>(y));
        else
            store_stream(reinterpret_cast<u32x4 *>(data + kNopeDim) + (lane - kRopeLane), pack_bf16x8<HW>(y));
    }
    if (lane == 0) {
        uint8_t *rec = base + (int64_t)a.block_size * kSlotData + (int64_t)sib * kSlotScale;
        if constexpr (SYS)
            store_sys2(rec, kSlotScale, 0u, u32x2{rec0, rec1});
        else
            store_stream2(reinterpret_cast<u32x2 *>(rec), u32x2{rec0, rec1});
    }
}

// The kv rows of tokens t0 .. t0+n-1 (n = a.kv_per_wave <= N) on one
// wavefront: every slot and row load is issued first, then the rows are
// finished one after another.  A token whose slot is out of range is skipped
// (wave-uniform) before its row is read.
template <bool HW, bool SYS, int N>
__device__ __forceinline__ void kv_rows(const KernelArgs &a, int64_t t0, uint32_t lane)
{
    int64_t slot[N];
    u32x4 d[N];
    // All N slot loads are issued before any is used: an index past the batch
    // is clamped to its last token (in bounds) and masked afterwards.  Loaded
    // under the per-token conditions instead, the compiler waited for each
    // slot before issuing the next (four round trips).  Issuing them together
    // is 0.2% faster at 32768x64 and 0.5-0.8% at 32768x8 and 8192x16, and
    // 0.3% slower at 2048x64 (41.35 -> 41.46 us), measured on MI355X.
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const int64_t t = t0 + u < a.num_tokens ? t0 + u : a.num_tokens - 1;
        slot[u] = a.slot_mapping[t];
    }
#pragma unroll
    for (int u = 0; u < N; ++u)
        if ((uint32_t)u >= a.kv_per_wave || t0 + u >= a.num_tokens)
            slot[u] = -1;
#pragma unroll
    for (int u = 0; u < N; ++u)
        if (slot[u] >= 0 && slot[u] < a.num_slots)
            d[u] = load_stream(reinterpret_cast<const u32x4 *>(a.kv + (t0 + u) * kHeadDim) + lane);
    float w[8];
    unpack_bf16x8(reinterpret_cast<const u32x4 *>(a.kv_w)[lane], w);
#pragma unroll
    for (int u = 0; u < N; ++u)
        if (slot[u] >= 0 && slot[u] < a.num_slots)
            kv_finish<HW, SYS>(a, t0 + u, slot[u], d[u], w, lane);
}

// ------------------------------------------------------------------ kernel

// kv workgroup `b` (its index among the kv workgroups): its wavefront takes
// a.kv_per_wave consecutive tokens' kv rows.
template <int U, bool HW>
__device__ __forceinline__ void kv_workgroup(const KernelArgs &a, int64_t b, uint32_t wave,
                                             uint32_t waves_per_block, uint32_t lane)
{
    const int64_t t = (b * waves_per_block + wave) * a.kv_per_wave;
    if (t < a.num_tokens)
        kv_rows<HW, U == 1, kMaxKvPerWave>(a, t, lane);
}

// q workgroup `b` (its index among the q workgroups): its wavefront takes one
// q row, or U heads of one token.
template <int U, bool HAS_W, bool HW>
__device__ __forceinline__ void q_workgroup(const KernelArgs &a, int64_t b, uint32_t wave,
                                            uint32_t waves_per_block, uint32_t lane)
{
    const int64_t wv = b * waves_per_block + wave;
    if constexpr (U == 1) {
        if (wv < a.q_rows)
            q_row<HAS_W, HW>(a, wv, lane);
    } else {
        if (wv < a.num_tokens * (int64_t)a.chunks)
            q_chunk<U, HAS_W, HW>(a, (uint32_t)wv, lane);
    }
}

// SPLIT: this dispatch is one of several covering a grid past 2^32
// work-items, so its workgroup indices start at a.block_base.  Single
// dispatches (every grid below about 2^26 q rows) use the instance without
// the offset: measured on MI355X, the always-on add cost 0.3-0.6% at
// 32768x64 and 131072x128.
template <int U, bool HAS_W, bool HW, bool SPLIT>
__global__ __launch_bounds__(512) void qkv_prep_kernel(KernelArgs a)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t waves_per_block = blockDim.x >> 6;
    const int64_t blk = SPLIT ? (int64_t)blockIdx.x + a.block_base : (int64_t)blockIdx.x;
    if constexpr (U == 2) {
        // Grid index -> kv or q workgroup and its index among those: kv first,
        // or kv workgroup j at index j * kv_period with the q workgroups in
        // the gaps and after (the grid has fewer than 2^31 workgroups there,
        // so the fixed-point division is exact).  One call site per body
        // keeps the instance's code size.
        bool kv = blk < a.kv_blocks;
        int64_t idx = kv ? blk : blk - a.kv_blocks;
        if (a.kv_period != 0) {
            const uint32_t j = fastdiv((uint32_t)blk, a.period_div);
            kv = j < a.kv_blocks && (uint32_t)blk == j * a.kv_period;
            idx = kv ? (int64_t)j : blk - (j < a.kv_blocks ? (int64_t)j + 1 : (int64_t)a.kv_blocks);
        }
        if (kv)
            kv_workgroup<U, HW>(a, idx, wave, waves_per_block, lane);
        else
            q_workgroup<U, HAS_W, HW>(a, idx, wave, waves_per_block, lane);
    } else {
        if (blk < a.kv_blocks)
            kv_workgroup<U, HW>(a, blk, wave, waves_per_block, lane);
        else
            q_workgroup<U, HAS_W, HW>(a, blk - a.kv_blocks, wave, waves_per_block, lane);
    }
}

template <int U, bool HAS_W, bool HW>
hipError_t launch_variant(const KernelArgs &a, bool split, dim3 grid, dim3 block, hipStream_t stream)
{
    if (split)
        hipLaunchKernelGGL((qkv_prep_kernel<U, HAS_W, HW, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((qkv_prep_kernel<U, HAS_W, HW, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <int U>
hipError_t launch_u(const KernelArgs &a, bool has_w, bool hw, bool split, dim3 grid, dim3 block, hipStream_t st)
{
    if (has_w)
        return hw ? launch_variant<U, true, true>(a, split, grid, block, st)
                  : launch_variant<U, true, false>(a, split, grid, block, st);
    return hw ? launch_variant<U, false, true>(a, split, grid, block, st)
              : launch_variant<U, false, false>(a, split, grid, block, st);
}

}  // namespace

hipError_t launch_qkv_prep(const KernelArgs &a, const LaunchShape &s, hipStream_t stream)
{
    const int64_t total = s.kv_blocks + s.q_blocks;
    const int64_t per = max_blocks_per_launch(s.waves_per_block);
    const dim3 block(64u * (uint32_t)s.waves_per_block);
    const bool has_w = a.q_w != nullptr;
    const bool hw = s.convert == 2;
    const bool split = total > per;
    for (int64_t base = 0; base < total; base += per) {
        KernelArgs k = a;
        k.block_base = base;
        const dim3 grid((uint32_t)(total - base < per ? total - base : per));
        hipError_t e;
        switch (s.rows_per_wave) {
        case 1: e = launch_u<1>(k, has_w, hw, split, grid, block, stream); break;
        case 2: e = launch_u<2>(k, has_w, hw, split, grid, block, stream); break;
        case 4: e = launch_u<4>(k, has_w, hw, split, grid, block, stream); break;
        default: e = hipErrorInvalidValue;
        }
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace qkvp
