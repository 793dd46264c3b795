// Launch arguments of the MXFP8 norm-quant kernel, shared between its host
// entry point (mxfp8_api.cpp) and mxfp8_norm_quant.hip.  Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
    int32_t padded_cols;
    float eps;
};

// Enqueue the kernel for hidden = 512 * K, K = 1..16 (checked by the caller).
hipError_t launch_mxfp8(const MxArgs &a, hipStream_t stream);

}  // namespace qkvp
