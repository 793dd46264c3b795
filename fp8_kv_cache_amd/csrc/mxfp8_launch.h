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

// Rows of up to kMxMaxGroups groups of 512 values (hidden <= 16384).
constexpr int kMxMaxGroups = 32;

// Enqueue the kernel for hidden a multiple of 128, 128 <= hidden <= 512 *
// kMxMaxGroups (checked by the caller).
hipError_t launch_mxfp8(const MxArgs &a, hipStream_t stream);

}  // namespace qkvp
