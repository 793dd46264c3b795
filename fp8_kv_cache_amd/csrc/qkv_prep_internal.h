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
constexpr int kRowsPerSet = 4;  // a wavefront works on 4 rows at once, 16 lanes each

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
    int64_t num_slots;         // num_blocks * block_size
    int64_t q_rows;            // T * H
    int64_t num_tokens;        // T
    int64_t q_sets;            // ceil(q_rows / 4)
    int64_t kv_sets;           // ceil(T / 4)
    uint32_t num_heads;
    uint32_t block_size;
    uint32_t kv_blocks;        // workgroups [0, kv_blocks) take kv sets
    float eps;
};

struct LaunchShape {
    int sets_per_wave;    // q sets per wavefront (1, 2, 4)
    int waves_per_block;  // 1, 2, 4, 8
    int convert;          // 1 integer rounding, 2 conversion instructions
    int64_t kv_blocks;
    int64_t q_blocks;
};

// Enqueue the kernel.  Returns the hipError_t of the launch.
hipError_t launch_qkv_prep(const KernelArgs &a, const LaunchShape &s, hipStream_t stream);

}  // namespace qkvp
