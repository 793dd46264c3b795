// Host side of the MXFP8 norm-quant entry points: the scale-buffer size, the
// argument checks and the launch.  Declarations and contracts:
// include/qkv_prep_mxfp8.h.
#include "qkv_prep.h"
#include "qkv_prep_mxfp8.h"

#include <cstdint>

#include "mxfp8_launch.h"
#include "qkv_prep_host.h"

namespace {

bool aligned16(const void *p) { return qkvp::aligned(p, 16); }

// The kernel indexes rows (padded to 128) in 32 bits.
constexpr int64_t kMaxRows = ((int64_t)1 << 31) - 128;

}  // namespace

extern "C" int64_t qkv_prep_mxfp8_scale_bytes(int64_t m, int32_t hidden)
{
    if (m < 0 || hidden <= 0 || hidden % 128)
        return -1;
    const int64_t cols = hidden / 32;            // a multiple of 4: no column padding
    if (m > INT64_MAX - 127)
        return -1;
    const int64_t rows_padded = (m + 127) / 128 * 128;
    if (rows_padded > INT64_MAX / cols)
        return -1;
    return rows_padded * cols;
}

extern "C" int qkv_prep_mxfp8_norm_quant(const qkv_prep_mxfp8_args *a, int device, void *stream)
{
    if (!a || a->m < 0 || !(a->eps >= 0.0f) || a->eps > 3.4e38f)
        return QKV_PREP_ERR_INVALID_ARG;
    if (a->hidden <= 0 || a->hidden % 128 || a->hidden > 512 * qkvp::kMxMaxGroups)
        return QKV_PREP_ERR_UNSUPPORTED;
    if (a->m == 0)
        return QKV_PREP_OK;
    if (!a->x || !a->gamma || !a->quant_out || !a->scale_out)
        return QKV_PREP_ERR_INVALID_ARG;
    if (!aligned16(a->x) || !aligned16(a->gamma) || !aligned16(a->quant_out) || !qkvp::aligned(a->scale_out, 4) ||
        (a->residual && !aligned16(a->residual)) || (a->residual_out && !aligned16(a->residual_out)))
        return QKV_PREP_ERR_MISALIGNED;
    if (a->m > kMaxRows)
        return QKV_PREP_ERR_UNSUPPORTED;
    const int64_t rows_padded = (a->m + 127) / 128 * 128;
    // One workgroup per padded row; the dispatch counts work-items in 32 bits.
    if (rows_padded * qkvp::mx_threads_per_row(a->hidden) >= ((int64_t)1 << 32))
        return QKV_PREP_ERR_UNSUPPORTED;
    qkvp::MxArgs k;
    k.x = static_cast<const uint16_t *>(a->x);
    k.residual = static_cast<const uint16_t *>(a->residual);
    k.residual_out = static_cast<uint16_t *>(a->residual_out);
    k.gamma = static_cast<const uint16_t *>(a->gamma);
    k.quant_out = static_cast<uint8_t *>(a->quant_out);
    k.scale_out = static_cast<uint8_t *>(a->scale_out);
    k.m = a->m;
    k.rows_padded = rows_padded;
    k.hidden = a->hidden;
    k.chunks = a->hidden / 8;
    k.padded_cols = a->hidden / 32;             // a multiple of 4: no column padding
    k.eps = a->eps;
    if (!qkvp::device_exists(device))
        return QKV_PREP_ERR_NO_DEVICE;
    qkvp::DeviceScope scope(device);
    if (!scope.ok())
        return QKV_PREP_ERR_NO_DEVICE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (qkvp::launch_mxfp8(k, st) != hipSuccess)
        return QKV_PREP_ERR_LAUNCH;
    static const bool sync = qkvp::env_flag("QKV_PREP_SYNC");
    if (sync && hipStreamSynchronize(st) != hipSuccess)
        return QKV_PREP_ERR_DEVICE;
    return QKV_PREP_OK;
}
