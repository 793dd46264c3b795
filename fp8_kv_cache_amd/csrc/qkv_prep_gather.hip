// Cache reader for the FP8 + UE8M0 paged cache written by qkv_prep_kernel:
// dequantize and gather slots back into fp32 or bf16 rows (the cache layout is
// the one stated in include/qkv_prep.h).  HBM bound: 584 bytes read and 1 or
// 2 KiB written per row; one wavefront per fp32 row or per two bf16 rows;
// non-temporal system-scope stores (plain loads: a slot's lines are shared
// with its neighbours).
#include "qkv_prep_gather.h"
#include "qkvp_device.h"

namespace qkvp {
namespace {

using namespace dev;

constexpr int kRopeLane = kNopeDim / 8;  // lanes 56..63 hold the rope chunks

// Four E4M3 codes (byte k of `codes` is dim k) times 2^(b - 127), b a scale
// byte 0..255, as v_ldexp_f32: the power is applied to the exponent, never
// formed as a float, so byte 255 (2^128, past the fp32 range) works like any
// other.  The results are exact (an E4M3 value has 4 significant bits, and the
// smallest product, 2^-9 * 2^-127, is an fp32 subnormal) except those of
// 2^128 and above, which only byte 255 reaches and which become infinity.
__device__ __forceinline__ u32x4 dequant4(uint32_t codes, uint32_t b)
{
    const int e = (int)b - 127;
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);
    return u32x4{__float_as_uint(__builtin_ldexpf(lo[0], e)), __float_as_uint(__builtin_ldexpf(lo[1], e)),
                 __float_as_uint(__builtin_ldexpf(hi[0], e)), __float_as_uint(__builtin_ldexpf(hi[1], e))};
}

// bf16 rows: R consecutive rows per wavefront.  Lane l < 56 reads the 8
// codes of dims 8l..8l+7 and the scale byte of their block; lanes 56..63 read
// 16 bytes of rope bf16; each lane stores its 16 output bytes, so one store
// covers a 1 KiB row.  All R rows' slot and data loads are issued before the
// first row is finished: the wavefront's two dependent round trips (slot,
// then data) are then shared by R rows.  Measured on MI355X over a
// 262144-slot block walk by graph replay: two rows per wavefront 59.6 us
// against 63.9 us for one (6.6 -> 7.1 TB/s); four or eight gain less.  fp32
// rows lose with the same change (92.3 -> 97.5 us at two rows), so they keep
// one row per wavefront.
template <int R>
__device__ __forceinline__ void gather_rows_bf16(const GatherArgs &a, int64_t i0, uint32_t lane)
{
    int64_t slot[R];
#pragma unroll
    for (int u = 0; u < R; ++u)
        slot[u] = i0 + u < a.n ? a.slots[i0 + u] : -1;
    u32x4 d[R];
    uint32_t b[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        d[u] = u32x4{0u, 0u, 0u, 0u};
        b[u] = 0u;
        if (slot[u] >= 0 && slot[u] < a.num_slots) {
            const uint32_t s32 = (uint32_t)slot[u];
            const uint32_t blk = fastdiv(s32, a.blocks);
            const uint32_t sib = s32 - blk * a.block_size;
            const uint8_t *base = a.cache + (int64_t)blk * a.block_size * kSlotBytes;
            const uint8_t *data = base + (int64_t)sib * kSlotData;
            if (lane < kRopeLane) {
                const u32x2 codes = *(reinterpret_cast<const u32x2 *>(data) + lane);
                d[u] = u32x4{codes[0], codes[1], 0u, 0u};
                b[u] = base[(int64_t)a.block_size * kSlotData + (int64_t)sib * kSlotScale + lane / 8];
            } else {
                d[u] = *(reinterpret_cast<const u32x4 *>(data + kNopeDim) + (lane - kRopeLane));
            }
        }
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
        if (i0 + u >= a.n)
            break;
        float v[8];
        if (slot[u] < 0 || slot[u] >= a.num_slots) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = 0.0f;
        } else if (lane < kRopeLane) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 q = dequant4(d[u][h], b[u]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[4 * h + e] = __uint_as_float(q[e]);
            }
        } else {
            unpack_bf16x8(d[u], v);
        }
        store_sys(static_cast<uint8_t *>(a.out) + (i0 + u) * 1024, 1024u, lane * 16u, pack_bf16x8<true>(v));
    }
}

// fp32 rows (2 KiB): lane l owns dims 4l..4l+3 and 256+4l..256+4l+3, so each
// of the wavefront's two 16-byte stores covers 1 KiB of the row contiguously.
// Dims 4l.. sit in quantization block l/16 (0..3); dims 256+4l.. in block
// 4 + l/16 for l < 48, and are rope dims 448 + 4(l - 48).. for l >= 48.  Every
// lane reads the slot's 8-byte scale record (one broadcast load).
__device__ __forceinline__ void gather_row_f32(const GatherArgs &a, int64_t i, uint32_t lane)
{
    const int64_t slot = a.slots[i];
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (slot >= 0 && slot < a.num_slots) {
        const uint32_t s32 = (uint32_t)slot;
        const uint32_t blk = fastdiv(s32, a.blocks);
        const uint32_t sib = s32 - blk * a.block_size;
        const uint8_t *base = a.cache + (int64_t)blk * a.block_size * kSlotBytes;
        const uint8_t *data = base + (int64_t)sib * kSlotData;
        const u32x2 rec = *reinterpret_cast<const u32x2 *>(base + (int64_t)a.block_size * kSlotData +
                                                          (int64_t)sib * kSlotScale);
        const uint32_t shift = 8u * (lane >> 4);
        lo = dequant4(reinterpret_cast<const uint32_t *>(data)[lane], (rec[0] >> shift) & 0xffu);
        if (lane < 48) {
            hi = dequant4(reinterpret_cast<const uint32_t *>(data + 256)[lane], (rec[1] >> shift) & 0xffu);
        } else {
            const u32x2 r = reinterpret_cast<const u32x2 *>(data + kNopeDim)[lane - 48];
            hi = u32x4{r[0] << 16, r[0] & 0xffff0000u, r[1] << 16, r[1] & 0xffff0000u};
        }
    }
    uint8_t *dst = static_cast<uint8_t *>(a.out) + i * 2048;
    store_sys(dst, 2048u, lane * 16u, lo);
    store_sys(dst, 2048u, 1024u + lane * 16u, hi);
}

// Workgroups are dispatched to the 8 XCDs round-robin, and each XCD has its
// own L2.  Rows next to each other in the slot list usually read neighbouring
// slots (a block-table walk reads a block's slots in order), which share cache
// lines: 8 scale records per 64-byte segment, and the 128-byte line where one
// slot's data ends and the next begins.  So workgroup b takes the rows of
// workgroup slot xcd_row_block(b, chunk): every XCD gets `chunk` consecutive
// workgroups' rows out of each window of 8 * chunk (a bijection of [0, grid)
// when grid is a multiple of 8 * chunk).
__device__ __forceinline__ uint32_t xcd_row_block(uint32_t b, uint32_t chunk)
{
    if (chunk == 0)
        return b;
    const uint32_t win = 8u * chunk, w = b / win, r = b - w * win;
    return w * win + (r & 7u) * chunk + (r >> 3);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(512) void gather_kernel(GatherArgs a)
{
    constexpr int R = OUT_BF16 ? kBf16Rows : kF32Rows;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t unit = (int64_t)xcd_row_block(blockIdx.x, a.xcd_chunk) * (blockDim.x >> 6) + wave;
    const int64_t i0 = unit * R;
    if (i0 < a.n) {
        if constexpr (OUT_BF16)
            gather_rows_bf16<R>(a, i0, lane);
        else
            gather_row_f32(a, i0, lane);
    }
}

}  // namespace

hipError_t launch_gather(const GatherArgs &a, int waves_per_block, hipStream_t stream)
{
    GatherArgs g = a;
    const GatherGrid gg = gather_grid(a.n, a.out_bf16 != 0, waves_per_block);
    g.xcd_chunk = gg.xcd_chunk;
    const dim3 grid((uint32_t)gg.blocks), block(64u * (uint32_t)waves_per_block);
    if (a.out_bf16)
        hipLaunchKernelGGL(gather_kernel<true>, grid, block, 0, stream, g);
    else
        hipLaunchKernelGGL(gather_kernel<false>, grid, block, 0, stream, g);
    return hipGetLastError();
}

}  // namespace qkvp
