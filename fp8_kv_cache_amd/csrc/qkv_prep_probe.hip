// The measurement and verification probes of libqkv_prep_probe.so (see
// include/qkv_prep_probe.h): a streaming copy and an in-place streaming update
// used as bandwidth ceilings, and the operators' own number-format code run on
// arrays so that tests can compare it with a reference on every input pattern.
// None of this is part of the operators; it is built into its own library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qkv_prep_probe.h"
#include "qkvp_device.h"

namespace {

using qkvp::dev::store_sys;
using qkvp::dev::u32x2;
using qkvp::dev::u32x4;
// One 16-byte non-temporal load and one 16-byte store per lane, 256-lane
// blocks: the fastest of the copy shapes measured on MI355X (1, 2, 4, 8 and 16
// loads per lane; 256, 512 and 1024 lanes per block; plain or non-temporal;
// natural or XCD-contiguous block order), about 6.4-6.5 TB/s at 0.5-4 GiB with
// non-temporal stores.  A sweep of the load and store cache-policy bits (sc0,
// sc1, nt) then found the non-temporal system-scope store (nt sc1) best, at
// ~6.7 TB/s; every load policy with nt set is within noise of the others.
constexpr int kUnroll = 1;
constexpr int kThreads = 256;

// Block b copies kUnroll * kThreads consecutive 16-byte units; all loads are
// issued before the first store.
__global__ __launch_bounds__(kThreads) void stream_copy(u32x4 *dst, const u32x4 *src, int64_t n)
{
    const int64_t first = (int64_t)blockIdx.x * (kThreads * kUnroll);
    const int64_t base = first + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kThreads;
        if (i < n)
            v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kThreads;
        if (i < n)
            store_sys(dst + first, kThreads * kUnroll * 16u, (uint32_t)(i - first) * 16u, v[u]);
    }
}

// In-place update, one 16-byte chunk per lane, one wavefront per workgroup.
// Measured on MI355X at 4 GiB: a store issued right after its load's data
// arrives streams at only ~4.5 TB/s; pausing the wavefront for a moment
// (s_sleep 2, ~128 cycles) between the load and the store gives ~6.7 TB/s,
// above the two-buffer copy.  A wave-wide reduction in the same place does not
// help (~4.5 TB/s); sleeps of 2 to 32 units are the same.  The nt sc1 store
// policy adds ~1.5% (~6.8 TB/s at 2 GiB).
constexpr int kUpdateThreads = 64;

__global__ __launch_bounds__(kUpdateThreads) void stream_update(u32x4 *buf, int64_t n)
{
    const int64_t first = (int64_t)blockIdx.x * kUpdateThreads;
    const int64_t i = first + threadIdx.x;
    if (i < n) {
        u32x4 v = __builtin_nontemporal_load(buf + i);
        v[0] += 1u;
        __builtin_amdgcn_s_sleep(2);
        store_sys(buf + first, kUpdateThreads * 16u, threadIdx.x * 16u, v);
    }
}

// The operator's conversions (qkvp::dev::pack_e4m3 / pack_bf16) on four
// values per thread.
template <bool HW>
__global__ __launch_bounds__(256) void convert_probe(const u32x4 *in, uint32_t *e4m3, u32x2 *bf16, int64_t quads)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= quads)
        return;
    const u32x4 v = in[i];
    const float f0 = __uint_as_float(v[0]), f1 = __uint_as_float(v[1]);
    const float f2 = __uint_as_float(v[2]), f3 = __uint_as_float(v[3]);
    if (e4m3)
        e4m3[i] = qkvp::dev::pack_e4m3<HW>(f0, f1, f2, f3);
    if (bf16)
        bf16[i] = u32x2{qkvp::dev::pack_bf16<HW>(f0, f1), qkvp::dev::pack_bf16<HW>(f2, f3)};
}

// The two UE8M0 rules on one value per thread: the main operator's scale
// byte of amax (qkvp::dev::ue8m0_exponent + 127) and the MXFP8 operator's byte
// (qkvp::dev::ue8m0_byte_up); thread i < 256 also writes the MXFP8 inverse
// scale of byte i.
__global__ __launch_bounds__(256) void ue8m0_probe(const float *in, int64_t n, uint8_t *op_byte, uint8_t *mx_byte,
                                                   float *mx_inverse)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (mx_inverse && i < 256)
        mx_inverse[i] = qkvp::dev::ue8m0_inverse_scale((uint32_t)i);
    if (i >= n)
        return;
    const float v = in[i];
    if (op_byte)
        op_byte[i] = (uint8_t)(qkvp::dev::ue8m0_exponent(__float_as_uint(v)) + 127);
    if (mx_byte)
        mx_byte[i] = (uint8_t)qkvp::dev::ue8m0_byte_up(v);
}

}  // namespace

extern "C" int qkv_prep_probe_convert(const float *in, int64_t n, void *e4m3_out, void *bf16_out, int32_t convert,
                                      void *stream)
{
    const uintptr_t pi = reinterpret_cast<uintptr_t>(in), pe = reinterpret_cast<uintptr_t>(e4m3_out),
                    pb = reinterpret_cast<uintptr_t>(bf16_out);
    if (n < 0 || (n & 3) || n >= ((int64_t)1 << 33) || (convert != 1 && convert != 2) || (pi & 15) ||
        (pe & 3) || (pb & 7) || (n > 0 && !in))
        return 1;
    if (n == 0)
        return 0;
    const int64_t quads = n / 4;
    const dim3 grid((uint32_t)((quads + 255) / 256)), block(256);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(in);
    uint32_t *e = static_cast<uint32_t *>(e4m3_out);
    u32x2 *b = static_cast<u32x2 *>(bf16_out);
    if (convert == 2)
        hipLaunchKernelGGL(convert_probe<true>, grid, block, 0, st, src, e, b, quads);
    else
        hipLaunchKernelGGL(convert_probe<false>, grid, block, 0, st, src, e, b, quads);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int qkv_prep_probe_update(void *buf, int64_t bytes, void *stream)
{
    if (bytes < 0 || (bytes > 0 && !buf) || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15))
        return 1;
    if (bytes == 0)
        return 0;
    const int64_t n = bytes / 16;
    const int64_t blocks = (n + kUpdateThreads - 1) / kUpdateThreads;
    if (blocks >= ((int64_t)1 << 31))
        return 1;
    hipLaunchKernelGGL(stream_update, dim3((uint32_t)blocks), dim3(kUpdateThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<u32x4 *>(buf), n);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int qkv_prep_probe_copy(void *dst, const void *src, int64_t bytes, void *stream)
{
    if (bytes < 0 || (bytes > 0 && (!dst || !src)) || (bytes & 15) ||
        (reinterpret_cast<uintptr_t>(dst) & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
        return 1;
    if (bytes == 0)
        return 0;
    const int64_t n = bytes / 16;
    const int64_t per_block = (int64_t)kThreads * kUnroll;
    const int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks >= ((int64_t)1 << 31))
        return 1;
    hipLaunchKernelGGL(stream_copy, dim3((uint32_t)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<u32x4 *>(dst),
                       static_cast<const u32x4 *>(src), n);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int qkv_prep_probe_ue8m0(const float *in, int64_t n, void *op_byte_out, void *mx_byte_out,
                                    void *mx_inverse_out, void *stream)
{
    if (n < 0 || n >= ((int64_t)1 << 38) || (n > 0 && !in) || (reinterpret_cast<uintptr_t>(in) & 3) ||
        (reinterpret_cast<uintptr_t>(mx_inverse_out) & 3))
        return 1;
    const int64_t threads = n > 256 ? n : 256;
    const int64_t blocks = mx_inverse_out ? (threads + 255) / 256 : (n + 255) / 256;
    if (blocks == 0)
        return 0;
    if (blocks >= ((int64_t)1 << 31))
        return 1;
    hipLaunchKernelGGL(ue8m0_probe, dim3((uint32_t)blocks), dim3(256), 0, static_cast<hipStream_t>(stream), in, n,
                       static_cast<uint8_t *>(op_byte_out), static_cast<uint8_t *>(mx_byte_out),
                       static_cast<float *>(mx_inverse_out));
    return hipGetLastError() == hipSuccess ? 0 : 5;
}
