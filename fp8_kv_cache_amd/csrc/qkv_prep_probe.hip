// The measurement and verification probes of libqkv_prep_probe.so (see
// include/qkv_prep_probe.h): policy-selectable read, write, copy and in-place
// update streams, two of which (a copy and an in-place update at their fastest
// settings) serve as bandwidth ceilings; the MXFP8 operator's memory access
// pattern without its arithmetic; and the operators' own number-format code
// run on arrays so that tests can compare it with a reference on every input
// pattern.  None of this is part of the operators; it is built into its own
// library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxfp8_launch.h"
#include "qkv_prep_probe.h"
#include "qkvp_device.h"

namespace {

using qkvp::dev::u32x2;
using qkvp::dev::u32x4;

// Policy-selectable streams (qkv_prep_probe_stream): 16-byte accesses, one or
// several per lane, blockDim.x lanes per workgroup, every access through a
// buffer descriptor whose base is the workgroup's first chunk, so any
// combination of the cache-policy bits can be put on the loads and on the
// stores.  These are the streams behind the read / write / copy / update rates,
// the cache-policy comparison and the rows-in-flight comparison quoted in the
// kernels' comments.
constexpr int kSc0 = 1, kNt = 2, kSc1 = 16;
enum StreamKind { kRead = 0, kWrite = 1, kCopy = 2, kUpdate = 3 };

template <int P>
__device__ __forceinline__ u32x4 load_policy(const u32x4 *base, uint32_t bytes, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(qkvp::dev::stream_rsrc(const_cast<u32x4 *>(base), bytes),
                                                  (int)off, 0, P);
}

template <int P>
__device__ __forceinline__ void store_policy(u32x4 *base, uint32_t bytes, uint32_t off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, qkvp::dev::stream_rsrc(base, bytes), (int)off, 0, P);
}

// LP / SP: the load / store policy bits.  SLEEP: the wavefront pauses
// (s_sleep 2, about 128 cycles) between its loads' arrival and its stores.
// DEPTH: each lane takes DEPTH chunks, blockDim.x chunks apart (with one
// wavefront per workgroup, DEPTH consecutive 1 KiB rows per wavefront), and
// issues all their loads before its first store.  The grid has exactly
// ceil(n / (blockDim.x * DEPTH)) workgroups, so every workgroup starts inside
// the range; the descriptor of each workgroup covers only its own chunks
// below n, so in the ragged last workgroup a load past n reads zeros and a
// store past n is dropped, with no memory access either way.  No access is
// guarded by a branch: guarded loads made the compiler wait for each load
// before issuing the next.  A read keeps its data live by comparing the XOR of
// each in-range chunk's four words with `key` and writing the key to the sink
// word dst[0] on a match.
template <int KIND, int LP, int SP, bool SLEEP, int DEPTH>
__device__ __forceinline__ void stream_body(u32x4 *dst, const u32x4 *src, int64_t n, uint32_t key,
                                            uint32_t xcd_chunk)
{
    // Workgroups go to the 8 XCDs round-robin (workgroup b to XCD b % 8).
    // With xcd_chunk > 0 (a grid of 8 * xcd_chunk workgroups), workgroup b
    // takes range (b % 8) * xcd_chunk + b / 8, so each XCD streams one
    // contiguous eighth; workgroups past the end exit before any access.
    const uint32_t b = xcd_chunk ? (blockIdx.x & 7u) * xcd_chunk + (blockIdx.x >> 3) : blockIdx.x;
    const int64_t per = (int64_t)blockDim.x * DEPTH;
    const int64_t first = (int64_t)b * per;
    if (first >= n)
        return;
    const int64_t left = n - first;
    const uint32_t span = (uint32_t)(left < per ? left : per) * 16u;
    uint32_t off[DEPTH];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u)
        off[u] = (u * blockDim.x + threadIdx.x) * 16u;
    if constexpr (KIND == kWrite) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            const int64_t i = first + off[u] / 16u;
            store_policy<SP>(dst + first, span, off[u], u32x4{(uint32_t)i, (uint32_t)(i >> 32), key, ~key});
        }
    } else {
        u32x4 v[DEPTH];
#pragma unroll
        for (int u = 0; u < DEPTH; ++u)
            v[u] = load_policy<LP>(KIND == kUpdate ? dst + first : src + first, span, off[u]);
        if constexpr (KIND == kRead) {
            bool hit = false;
#pragma unroll
            for (int u = 0; u < DEPTH; ++u)
                hit |= (off[u] < span) & ((v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]) == key);
            if (hit)
                *reinterpret_cast<uint32_t *>(dst) = key;
        } else {
            if constexpr (KIND == kUpdate) {
#pragma unroll
                for (int u = 0; u < DEPTH; ++u)
                    v[u][0] += 1u;
            }
            if constexpr (SLEEP)
                __builtin_amdgcn_s_sleep(2);
#pragma unroll
            for (int u = 0; u < DEPTH; ++u)
                store_policy<SP>(dst + first, span, off[u], v[u]);
        }
    }
}

template <int KIND, int LP, int SP, bool SLEEP, int DEPTH>
__global__ __launch_bounds__(1024) void policy_stream(u32x4 *dst, const u32x4 *src, int64_t n, uint32_t key,
                                                     uint32_t xcd_chunk)
{
    stream_body<KIND, LP, SP, SLEEP, DEPTH>(dst, src, n, key, xcd_chunk);
}

// The two ceilings are the policy streams at their fastest settings in the
// streams sweep (bench.py --mode streams, 512 MiB and 2 GiB buffers on
// MI355X): one wavefront per workgroup, non-temporal loads, nt sc1 stores.
// Copy: 6.80 TB/s with 64 lanes per workgroup, 6.67 with 256 and 6.29-6.49
// with 1024.  In-place update: 6.83-6.88 TB/s, the same with or without a
// pause before the store; 6.64-6.67 with 256 lanes.  They keep kernels of
// their own so that a profile can tell them apart.
constexpr int kCeilingLanes = 64;

__global__ __launch_bounds__(kCeilingLanes) void stream_copy(u32x4 *dst, const u32x4 *src, int64_t n, uint32_t key)
{
    stream_body<kCopy, kNt, kNt | kSc1, false, 1>(dst, src, n, key, 0u);
}

__global__ __launch_bounds__(kCeilingLanes) void stream_update(u32x4 *dst, const u32x4 *src, int64_t n, uint32_t key)
{
    stream_body<kUpdate, kNt, kNt | kSc1, false, 1>(dst, src, n, key, 0u);
}

struct StreamLaunch {
    dim3 grid, block;
    hipStream_t stream;
    u32x4 *dst;
    const u32x4 *src;
    int64_t n;
    uint32_t key;
    uint32_t xcd_chunk;
};

template <int KIND, int LP, int SP, bool SLEEP, int DEPTH = 1>
bool launch_stream(const StreamLaunch &L)
{
    hipLaunchKernelGGL((policy_stream<KIND, LP, SP, SLEEP, DEPTH>), L.grid, L.block, 0, L.stream, L.dst, L.src,
                       L.n, L.key, L.xcd_chunk);
    return true;
}

// Several chunks per lane: only with the fastest policies (nt loads, nt sc1
// stores) and no pause.
template <int DEPTH>
bool launch_deep(int kind, const StreamLaunch &L)
{
    switch (kind) {
    case kRead: return launch_stream<kRead, kNt, 0, false, DEPTH>(L);
    case kWrite: return launch_stream<kWrite, 0, kNt | kSc1, false, DEPTH>(L);
    case kCopy: return launch_stream<kCopy, kNt, kNt | kSc1, false, DEPTH>(L);
    case kUpdate: return launch_stream<kUpdate, kNt, kNt | kSc1, false, DEPTH>(L);
    default: return false;
    }
}

// The accepted policies: loads plain, nt or nt sc1; stores plain, nt, sc1,
// nt sc1 or sc0 nt sc1.  Anything else returns false (nothing launched).
template <int KIND, int LP, bool SLEEP>
bool launch_by_store(const StreamLaunch &L, int sp)
{
    switch (sp) {
    case 0: return launch_stream<KIND, LP, 0, SLEEP>(L);
    case kNt: return launch_stream<KIND, LP, kNt, SLEEP>(L);
    case kSc1: return launch_stream<KIND, LP, kSc1, SLEEP>(L);
    case kNt | kSc1: return launch_stream<KIND, LP, kNt | kSc1, SLEEP>(L);
    case kSc0 | kNt | kSc1: return launch_stream<KIND, LP, kSc0 | kNt | kSc1, SLEEP>(L);
    default: return false;
    }
}

template <int KIND, bool SLEEP>
bool launch_by_load(const StreamLaunch &L, int lp, int sp)
{
    switch (lp) {
    case 0: return launch_by_store<KIND, 0, SLEEP>(L, sp);
    case kNt: return launch_by_store<KIND, kNt, SLEEP>(L, sp);
    case kNt | kSc1: return launch_by_store<KIND, kNt | kSc1, SLEEP>(L, sp);
    default: return false;
    }
}

bool launch_policy_stream(int kind, int lp, int sp, bool sleep, const StreamLaunch &L)
{
    switch (kind) {
    case kRead:
        switch (lp) {
        case 0: return launch_stream<kRead, 0, 0, false>(L);
        case kNt: return launch_stream<kRead, kNt, 0, false>(L);
        case kNt | kSc1: return launch_stream<kRead, kNt | kSc1, 0, false>(L);
        default: return false;
        }
    case kWrite:
        switch (sp) {
        case 0: return launch_stream<kWrite, 0, 0, false>(L);
        case kNt: return launch_stream<kWrite, 0, kNt, false>(L);
        case kSc1: return launch_stream<kWrite, 0, kSc1, false>(L);
        case kNt | kSc1: return launch_stream<kWrite, 0, kNt | kSc1, false>(L);
        case kSc0 | kNt | kSc1: return launch_stream<kWrite, 0, kSc0 | kNt | kSc1, false>(L);
        default: return false;
        }
    case kCopy:
        return sleep ? launch_by_load<kCopy, true>(L, lp, sp) : launch_by_load<kCopy, false>(L, lp, sp);
    case kUpdate:
        return sleep ? launch_by_load<kUpdate, true>(L, lp, sp) : launch_by_load<kUpdate, false>(L, lp, sp);
    default: return false;
    }
}

bool valid_load_policy(int p) { return p == 0 || p == kNt || p == (kNt | kSc1); }
bool valid_store_policy(int p)
{
    return p == 0 || p == kNt || p == kSc1 || p == (kNt | kSc1) || p == (kSc0 | kNt | kSc1);
}

// The MXFP8 operator's memory access pattern with no arithmetic
// (qkv_prep_probe_mxfp8_pattern): its grid (one workgroup per row padded to
// 128 rows, G groups of 64 16-byte chunks per wavefront), its non-temporal
// loads of x and the residual, its nt sc1 stores of the residual output (16
// bytes per lane), its one LDS barrier where a row spans several wavefronts,
// then per group a 16-byte load of gamma (cache-resident) followed by that
// group's nt sc1 code store (8 bytes per lane) and 4-byte scale word from the
// first lane of each 16-lane row into the 128x4 swizzled layout, and the zero
// words of the padding rows.  The stored values are XORs of the loaded words,
// which keeps every load live and orders each group's stores after its gamma
// load, as in the operator.
struct MxPattern {
    const u32x4 *x;
    const u32x4 *residual;
    const u32x4 *gamma;
    uint8_t *residual_out;
    uint8_t *codes;
    uint8_t *scales;
    int64_t m;
    int32_t hidden;
    int32_t padded_cols;
};

template <int G, bool RES, bool CODES, bool SCALES, bool BARRIER>
__global__ __launch_bounds__(1024) void mxfp8_pattern(MxPattern a)
{
    __shared__ uint32_t wave_word[16];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = blockIdx.x;
    if (row >= a.m) {
        if constexpr (SCALES)
            for (int c = threadIdx.x * 4; c < a.padded_cols; c += blockDim.x * 4)
                *reinterpret_cast<uint32_t *>(a.scales + qkvp::mx_swizzled_offset(row, c, a.padded_cols)) = 0u;
        return;
    }
    const int64_t chunks_per_row = a.hidden / 8;
    u32x4 p[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int64_t chunk = (int64_t)(w * G + j) * 64 + lane;
        p[j] = qkvp::dev::load_stream(a.x + row * chunks_per_row + chunk);
        if constexpr (RES)
            p[j] ^= qkvp::dev::load_stream(a.residual + row * chunks_per_row + chunk);
    }
    if constexpr (RES) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint32_t chunk = (w * G + j) * 64 + lane;
            qkvp::dev::store_sys(a.residual_out + row * a.hidden * 2, (uint32_t)a.hidden * 2u, chunk * 16u, p[j]);
        }
    }
    uint32_t extra = 0;
    if constexpr (BARRIER) {
        if (lane == 0)
            wave_word[w] = p[0][0];
        __syncthreads();
        extra = wave_word[0];
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint32_t chunk = (w * G + j) * 64 + lane;
        if constexpr (CODES || SCALES) {
            const u32x4 gm = a.gamma[chunk];
            if constexpr (CODES)
                qkvp::dev::store_sys2(a.codes + row * a.hidden, (uint32_t)a.hidden, chunk * 8u,
                                      u32x2{p[j][0] ^ p[j][1] ^ gm[0] ^ extra, p[j][2] ^ p[j][3] ^ gm[1]});
            if constexpr (SCALES) {
                if ((lane & 15) == 0)
                    *reinterpret_cast<uint32_t *>(a.scales + qkvp::mx_swizzled_offset(row, chunk >> 2, a.padded_cols)) =
                        p[j][0] ^ p[j][3] ^ gm[3] ^ extra;
            }
        }
    }
}

template <int G, bool RES, bool CODES, bool SCALES>
void launch_mx_pattern_b(const MxPattern &a, bool barrier, dim3 grid, dim3 block, hipStream_t st)
{
    if (barrier)
        hipLaunchKernelGGL((mxfp8_pattern<G, RES, CODES, SCALES, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((mxfp8_pattern<G, RES, CODES, SCALES, false>), grid, block, 0, st, a);
}

template <int G>
void launch_mx_pattern(const MxPattern &a, int streams, dim3 grid, dim3 block, hipStream_t st)
{
    const bool barrier = (streams & 8) != 0;
    switch (streams & 7) {
    case 1: launch_mx_pattern_b<G, true, false, false>(a, barrier, grid, block, st); break;
    case 2: launch_mx_pattern_b<G, false, true, false>(a, barrier, grid, block, st); break;
    case 3: launch_mx_pattern_b<G, true, true, false>(a, barrier, grid, block, st); break;
    case 4: launch_mx_pattern_b<G, false, false, true>(a, barrier, grid, block, st); break;
    case 5: launch_mx_pattern_b<G, true, false, true>(a, barrier, grid, block, st); break;
    case 6: launch_mx_pattern_b<G, false, true, true>(a, barrier, grid, block, st); break;
    default: launch_mx_pattern_b<G, true, true, true>(a, barrier, grid, block, st); break;
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

static int ceiling_stream(int kind, void *dst, const void *src, int64_t bytes, hipStream_t stream)
{
    const int64_t n = bytes / 16;
    const int64_t blocks = (n + kCeilingLanes - 1) / kCeilingLanes;
    if (blocks >= ((int64_t)1 << 31))
        return 1;
    const dim3 grid((uint32_t)blocks), block(kCeilingLanes);
    u32x4 *d = static_cast<u32x4 *>(dst);
    const u32x4 *s = static_cast<const u32x4 *>(src);
    if (kind == kCopy)
        hipLaunchKernelGGL(stream_copy, grid, block, 0, stream, d, s, n, 0u);
    else
        hipLaunchKernelGGL(stream_update, grid, block, 0, stream, d, s, n, 0u);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int qkv_prep_probe_update(void *buf, int64_t bytes, void *stream)
{
    if (bytes < 0 || (bytes > 0 && !buf) || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15))
        return 1;
    if (bytes == 0)
        return 0;
    return ceiling_stream(kUpdate, buf, nullptr, bytes, static_cast<hipStream_t>(stream));
}

extern "C" int qkv_prep_probe_copy(void *dst, const void *src, int64_t bytes, void *stream)
{
    if (bytes < 0 || (bytes > 0 && (!dst || !src)) || (bytes & 15) ||
        (reinterpret_cast<uintptr_t>(dst) & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
        return 1;
    if (bytes == 0)
        return 0;
    return ceiling_stream(kCopy, dst, src, bytes, static_cast<hipStream_t>(stream));
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

extern "C" int qkv_prep_probe_stream(int32_t kind, int32_t load_policy, int32_t store_policy, int32_t sleep,
                                     int32_t lanes_per_block, int32_t depth, int32_t xcd_order, void *dst,
                                     const void *src, int64_t bytes, uint32_t key, void *stream)
{
    const uintptr_t pd = reinterpret_cast<uintptr_t>(dst), ps = reinterpret_cast<uintptr_t>(src);
    const bool reads = kind == kRead || kind == kCopy || kind == kUpdate;
    const bool writes = kind == kWrite || kind == kCopy || kind == kUpdate;
    if (kind < kRead || kind > kUpdate || bytes < 0 || (bytes & 15) || (sleep != 0 && sleep != 1))
        return 1;
    if (lanes_per_block != 64 && lanes_per_block != 128 && lanes_per_block != 256 && lanes_per_block != 512 &&
        lanes_per_block != 1024)
        return 1;
    if (reads ? !valid_load_policy(load_policy) : load_policy != 0)
        return 1;
    if (writes ? !valid_store_policy(store_policy) : store_policy != 0)
        return 1;
    if (sleep && kind != kCopy && kind != kUpdate)
        return 1;
    if (depth != 1 && depth != 2 && depth != 4 && depth != 8 && depth != 16)
        return 1;
    if (xcd_order != 0 && xcd_order != 1)
        return 1;
    if (depth > 1 && (sleep || load_policy != (reads ? kNt : 0) || store_policy != (writes ? (kNt | kSc1) : 0)))
        return 1;
    // dst: the sink word of a read (4-byte aligned), else the written range
    // (16-byte aligned); src: the range a read or copy loads, NULL otherwise.
    const bool needs_src = kind == kRead || kind == kCopy;
    if (!dst || (pd & (kind == kRead ? 3 : 15)) || (needs_src ? (!src || (ps & 15)) : src != nullptr))
        return 1;
    if (kind == kCopy && bytes > 0 && pd < ps + (uint64_t)bytes && ps < pd + (uint64_t)bytes)
        return 1;
    if (bytes == 0)
        return 0;
    const int64_t n = bytes / 16;
    const int64_t per = (int64_t)lanes_per_block * depth;
    const int64_t blocks = (n + per - 1) / per;
    const int64_t chunk = xcd_order ? (blocks + 7) / 8 : 0;
    const int64_t grid = xcd_order ? 8 * chunk : blocks;
    if (grid >= ((int64_t)1 << 31))
        return 1;
    StreamLaunch L;
    L.grid = dim3((uint32_t)grid);
    L.xcd_chunk = (uint32_t)chunk;
    L.block = dim3((uint32_t)lanes_per_block);
    L.stream = static_cast<hipStream_t>(stream);
    L.dst = static_cast<u32x4 *>(dst);
    L.src = static_cast<const u32x4 *>(src);
    L.n = n;
    L.key = key;
    bool launched;
    switch (depth) {
    case 2: launched = launch_deep<2>(kind, L); break;
    case 4: launched = launch_deep<4>(kind, L); break;
    case 8: launched = launch_deep<8>(kind, L); break;
    case 16: launched = launch_deep<16>(kind, L); break;
    default: launched = launch_policy_stream(kind, load_policy, store_policy, sleep != 0, L);
    }
    if (!launched)
        return 1;
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int qkv_prep_probe_mxfp8_pattern(const void *x, const void *residual, const void *gamma,
                                            void *residual_out, void *codes, void *scales, int64_t m,
                                            int32_t hidden, int32_t streams, void *stream)
{
    const bool res = streams & 1, cod = streams & 2, sca = streams & 4;
    if (streams < 1 || streams > 15 || !(streams & 7) || m < 0 || hidden < 512 || hidden % 512 ||
        hidden > 512 * qkvp::kMxMaxGroups)
        return 1;
    const int k = hidden / 512;
    if (!qkvp::mx_launchable(k))
        return 1;
    auto misaligned = [](const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
    if (!x || misaligned(x, 16) || (res && (!residual || !residual_out || misaligned(residual, 16) ||
                                           misaligned(residual_out, 16))) ||
        (cod && (!codes || misaligned(codes, 8))) || (sca && (!scales || misaligned(scales, 4))) ||
        ((cod || sca) && (!gamma || misaligned(gamma, 16))))
        return 1;
    const int64_t rows_padded = (m + 127) / 128 * 128;
    const int g = qkvp::mx_groups_per_wave(k);
    const int64_t threads = 64 * (k / g);
    if (rows_padded * threads >= ((int64_t)1 << 32))
        return 1;
    if (rows_padded == 0)
        return 0;
    MxPattern a;
    a.x = static_cast<const u32x4 *>(x);
    a.residual = static_cast<const u32x4 *>(residual);
    a.gamma = static_cast<const u32x4 *>(gamma);
    a.residual_out = static_cast<uint8_t *>(residual_out);
    a.codes = static_cast<uint8_t *>(codes);
    a.scales = static_cast<uint8_t *>(scales);
    a.m = m;
    a.hidden = hidden;
    a.padded_cols = hidden / 32;
    const dim3 grid((uint32_t)rows_padded), block((uint32_t)threads);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (g == 2)
        launch_mx_pattern<2>(a, streams, grid, block, st);
    else
        launch_mx_pattern<1>(a, streams, grid, block, st);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}
