// Division by a launch-constant divisor with a multiply and a shift, for the
// index arithmetic of bandwidth-bound kernels (plain C++, shared by host and
// device code).
//
// For 1 <= d < 2^31, s = ceil(log2 d) and m = ceil(2^(32+s) / d), every
// numerator n < 2^32 satisfies n / d == (n * m) >> (32 + s) (the round-up
// method of Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994). m < 2^33, so for n < 2^31 the product fits in 64
// bits; callers keep numerators below 2^31.
#pragma once

#include <stdint.h>

namespace attnblk {

struct FastDiv {
    uint64_t m;
    uint32_t s;
};

inline FastDiv make_fast_div(uint32_t d) {
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    const uint64_t p = 1ull << (32 + s);
    return FastDiv{(p + d - 1) / d, s};
}

}  // namespace attnblk
