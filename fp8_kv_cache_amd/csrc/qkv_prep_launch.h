// The operator kernel's launch arguments and shape, shared between the host
// API (qkv_prep_api.cpp) and qkv_prep_kernels.hip.  Not part of the public ABI.
#pragma once

#include "qkv_prep_internal.h"

namespace qkvp {

struct KernelArgs {
    uint16_t *q;
    const uint16_t *kv;
    const uint16_t *q_w;       // may be null (weightless q norm)
    const uint16_t *kv_w;
    const int64_t *positions;
    const float *cos_sin;
    const int64_t *slot_mapping;
    uint8_t *cache;
    int64_t max_position;
    int64_t num_slots;         // num_blocks * block_size (< 2^31)
    int64_t q_rows;            // T * H (< 2^31)
    int64_t num_tokens;        // T
    uint32_t block_size;
    uint32_t kv_blocks;        // workgroups [0, kv_blocks) take kv rows
    uint32_t kv_per_wave;      // consecutive tokens' kv rows per wavefront (1, 2 or 4)
    FastDiv heads;             // divides a q row index by H
    FastDiv blocks;            // divides a slot by block_size
    uint32_t num_heads;        // H
    uint32_t chunks;           // q wavefronts per token: ceil(H / rows_per_wave)
    FastDiv chunk_div;         // divides a q wavefront index by `chunks`
    float eps;
    int32_t bf16_store;        // 1: kv slots are 1024 bytes of bf16, no quantization
    int64_t block_base;        // workgroup index of this dispatch's first workgroup
    uint32_t kv_period;        // 0: the kv workgroups come first; else kv workgroup j sits at
                               // grid index j * kv_period (two-heads instance only)
    FastDiv period_div;        // divides a grid index by kv_period
};

// The most consecutive tokens whose kv rows one wavefront takes.
constexpr int kMaxKvPerWave = 4;

struct LaunchShape {
    int rows_per_wave;    // q rows per wavefront (1; or 2, 4 heads of one token)
    int waves_per_block;  // 1, 2, 4, 8
    int convert;          // 1 integer rounding, 2 conversion instructions
    int kv_per_wave;      // tokens' kv rows per kv wavefront (1, 2, 4)
    int64_t kv_blocks;
    int64_t q_blocks;
    int64_t kv_period;    // 0, or the spacing of the kv workgroups in the grid (odd, >= 3)
};

// The most workgroups of `waves_per_block` wavefronts one dispatch takes: the
// dispatch counts work-items in 32 bits.  A larger grid is enqueued as
// consecutive dispatches of the same kernel, each covering the next range of
// workgroup indices (KernelArgs::block_base).
inline int64_t max_blocks_per_launch(int waves_per_block)
{
    return (((int64_t)1 << 32) - 1) / (64 * (int64_t)waves_per_block);
}

// Dispatches for a grid of `blocks` workgroups.
inline int64_t launches_for(int64_t blocks, int waves_per_block)
{
    const int64_t per = max_blocks_per_launch(waves_per_block);
    return (blocks + per - 1) / per;
}

// Enqueue the kernel (launches_for(...) dispatches, in order, on `stream`).
// Returns the hipError_t of the first launch that fails, else hipSuccess.
hipError_t launch_qkv_prep(const KernelArgs &a, const LaunchShape &s, hipStream_t stream);

}  // namespace qkvp
