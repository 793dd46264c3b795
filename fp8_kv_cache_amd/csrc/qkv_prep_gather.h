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
    uint32_t xcd_chunk;        // consecutive workgroups per XCD chunk (0: plain order); gather_grid sets it
};

// Rows per wavefront of each output type.
constexpr int kBf16Rows = 2;
constexpr int kF32Rows = 1;

// The reader's grid for n rows: workgroups of `waves_per_block` wavefronts,
// and the XCD chunking of the workgroup order.  Chunks of 64 rows (a cache
// block's worth of slots at the usual block size), counted in workgroups of
// rows_per_wave * waves_per_block rows, pad the grid to whole windows of
// 8 chunks.  Measured on MI355X over a 262144-slot block-table walk: fp32
// rows 6.5 -> 7.1 TB/s, bf16 rows 6.0 -> 6.3 TB/s; every slot in a random
// order: +2.5%.  Small grids keep the plain order (the padding would cost
// more), and so does a grid that the padding would take to 2^32 work-items
// or more (the dispatch counts work-items in 32 bits): with n < 2^26 the
// plain order always fits.
struct GatherGrid {
    int64_t blocks;
    uint32_t xcd_chunk;  // 0: plain order
};

inline GatherGrid gather_grid(int64_t n, bool out_bf16, int waves_per_block)
{
    const int rows = out_bf16 ? kBf16Rows : kF32Rows;
    const int64_t waves = (n + rows - 1) / rows;
    GatherGrid g{(waves + waves_per_block - 1) / waves_per_block, 0u};
    const int64_t rows_per_block = (int64_t)rows * waves_per_block;
    const uint32_t chunk = g.blocks * rows_per_block >= 4096 ? (uint32_t)(64 / rows_per_block) : 0u;
    if (chunk) {
        const int64_t padded = (g.blocks + 8 * chunk - 1) / (8 * chunk) * (8 * chunk);
        if (padded * 64 * waves_per_block < ((int64_t)1 << 32)) {
            g.blocks = padded;
            g.xcd_chunk = chunk;
        }
    }
    return g;
}

// Enqueue the cache reader: one wavefront per fp32 row or per two bf16 rows,
// `waves_per_block` wavefronts per workgroup, on the grid of gather_grid.
hipError_t launch_gather(const GatherArgs &a, int waves_per_block, hipStream_t stream);

}  // namespace qkvp
