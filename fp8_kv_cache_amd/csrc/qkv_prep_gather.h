// The cache reader's launch arguments, shared between the host API
// (qkv_prep_api.cpp) and qkv_prep_gather.hip.  Not part of the public ABI.
#pragma once

#include "qkv_prep_internal.h"

namespace qkvp {

struct GatherArgs {
    const uint8_t *cache;
    const int64_t *slots;
    void *out;
    int64_t num_slots;         // num_blocks * block_size (< 2^31)
    int64_t n;                 // rows to read
    uint32_t block_size;
    FastDiv blocks;
    int32_t out_bf16;          // 0: fp32 rows, 1: bf16 rows
    uint32_t xcd_chunk;        // consecutive workgroups per XCD chunk (0: plain order)
};

// Enqueue the cache reader: one wavefront per fp32 row or per two bf16 rows,
// `waves_per_block` wavefronts per workgroup.
hipError_t launch_gather(const GatherArgs &a, int waves_per_block, hipStream_t stream);

}  // namespace qkvp
