// Unsigned 32-bit division by a divisor fixed for a whole launch, as one
// multiply-high, one subtract, one add and two shifts (Granlund and
// Montgomery, "Division by Invariant Integers using Multiplication", PLDI
// 1994, section 4, the round-up method for N = 32-bit operands):
//   l = ceil(log2 d),  m = floor(2^32 (2^l - d) / d) + 1   (m < 2^32)
//   t = mulhi(m, n),   q = (t + ((n - t) >> 1)) >> (l - 1)     (l >= 1)
// exact for every 0 <= n < 2^32 and 1 <= d < 2^32; d = 1 keeps n.
// The host builds the constants; kernels evaluate them.  Plain C++ so a host
// compiler can build the same code for its test.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FGQ_HD __host__ __device__
#else
#define FGQ_HD
#endif

namespace fgq {

struct FastDiv {
    uint32_t d;      // divisor
    uint32_t m;      // multiplier
    uint32_t s;      // l - 1 (unused when d == 1)
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f{d, 0u, 0u};
    if (d <= 1) return f;
    uint32_t l = 0;
    while (l < 32 && (1ull << l) < d) ++l;   // l = ceil(log2 d), 1 <= l <= 32
    f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    f.s = l - 1;
    return f;
}

FGQ_HD inline uint32_t fastdiv(uint32_t n, const FastDiv &f) {
    if (f.d == 1) return n;
    const uint32_t t = (uint32_t)(((uint64_t)f.m * n) >> 32);
    return (t + ((n - t) >> 1)) >> f.s;
}

}  // namespace fgq
