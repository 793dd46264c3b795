// Launch arguments of the MXFP8 norm-quant kernel, shared between its host
// entry point (mxfp8_api.cpp) and mxfp8_norm_quant.hip.  Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace qkvp {

struct MxArgs {
    const uint16_t *x;
    const uint16_t *residual;
    uint16_t *residual_out;
    const uint16_t *gamma;
    uint8_t *quant_out;
    uint8_t *scale_out;
    int64_t m;
    int64_t rows_padded;
    int32_t hidden;
    int32_t chunks;            // hidden / 8: 16-byte chunks per row
    int32_t padded_cols;
    float eps;
};

// The byte of scale column `col` of row `row` in the 128x4 swizzled layout
// (rows in tiles of 128, each tile padded_cols * 128 bytes: column group
// col/4 takes 512 bytes, row r of the tile sits at (r % 32) * 16 + (r / 32) * 4
// in it, and the 4 columns of the group are consecutive bytes).
__host__ __device__ __forceinline__ int64_t mx_swizzled_offset(int64_t row, int64_t col, int64_t padded_cols)
{
    return (col & 3) + (col >> 2) * 512 + (row & 31) * 16 + ((row & 127) >> 5) * 4 + (row >> 7) * 128 * padded_cols;
}

// Rows of up to kMxMaxGroups groups of 512 values (hidden <= 16384).
constexpr int kMxMaxGroups = 32;

// Groups of 64 chunks per wavefront for a row of K groups.  Measured on
// MI355X at hidden 1024-8192 (two interleaved rounds): two groups per
// wavefront (K/2 wavefronts per row) is the fastest or tied everywhere; one
// group per wavefront is within 2%; one wavefront per row loses up to 60% at
// large K (VGPR pressure).  Odd K up to 15 uses one group per wavefront; an
// odd K above 16 is launched as K + 1 groups (the last one empty, which adds
// zeros to the sum) so that a workgroup stays within 16 wavefronts.
constexpr int mx_groups_per_wave(int K) { return K % 2 == 0 ? 2 : 1; }
constexpr bool mx_launchable(int K) { return K <= 16 || K % 2 == 0; }

// The groups a row of `hidden` values is launched with (hidden a positive
// multiple of 128, at most 512 * kMxMaxGroups), and the workgroup size: one
// workgroup per row, 64 lanes per wavefront.
constexpr int mx_launch_groups(int hidden)
{
    return mx_launchable((hidden + 511) / 512) ? (hidden + 511) / 512 : (hidden + 511) / 512 + 1;
}
constexpr int mx_threads_per_row(int hidden)
{
    return 64 * (mx_launch_groups(hidden) / mx_groups_per_wave(mx_launch_groups(hidden)));
}

// Enqueue the kernel for hidden a multiple of 128, 128 <= hidden <= 512 *
// kMxMaxGroups (checked by the caller).
hipError_t launch_mxfp8(const MxArgs &a, hipStream_t stream);

}  // namespace qkvp
