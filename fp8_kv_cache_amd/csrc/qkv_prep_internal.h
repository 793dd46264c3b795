// Constants of the cache layout and the fixed-point divider, shared by the
// host API and every kernel of the library.  Not part of the public ABI.
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

}  // namespace qkvp
