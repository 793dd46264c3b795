// Shared between the host API (qkv_prep_api.cpp) and the kernels
// (qkv_prep_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkvp {

constexpr int kHeadDim = 512;
constexpr int kNopeDim = 448;
constexpr int kRopeDim = 64;
constexpr int kSlotData = 576;
constexpr int kSlotScale = 8;
constexpr int kSlotBytes = 584;

// Unsigned division by a fixed divisor d >= 1 for dividends n < 2^31:
// n / d == (umulhi(n, mul) + n) >> shift, with shift = ceil(log2 d) and
// mul = floor(2^32 (2^shift - d) / d) + 1 (the round-up method of Granlund
// and Montgomery; n < 2^31 keeps umulhi + n inside 32 bits).
struct FastDiv {
    uint32_t mul;
    uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while ((1ull << l) < d)
        ++l;
    const uint64_t m = ((((uint64_t)1 << 32) * ((1ull << l) - d)) / d) + 1;
    return FastDiv{(uint32_t)m, l};
}

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
    FastDiv heads;             // divides a q row index by H
    FastDiv blocks;            // divides a slot by block_size
    float eps;
    int32_t bf16_store;        // 1: kv slots are 1024 bytes of bf16, no quantization
};

struct LaunchShape {
    int rows_per_wave;    // q rows per wavefront (1, 2, 4)
    int waves_per_block;  // 1, 2, 4, 8
    int convert;          // 1 integer rounding, 2 conversion instructions
    int64_t kv_blocks;
    int64_t q_blocks;
};

// Enqueue the kernel.  Returns the hipError_t of the launch.
hipError_t launch_qkv_prep(const KernelArgs &a, const LaunchShape &s, hipStream_t stream);

}  // namespace qkvp
