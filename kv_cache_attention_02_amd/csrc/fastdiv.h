// Division of a non-negative 32-bit integer by a divisor fixed for a whole
// launch, as one multiply-high, one add and one shift (Granlund and
// Montgomery, "Division by Invariant Integers using Multiplication", PLDI
// 1994, section 4, unsigned division): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1,
//     floor(n / d) = (mulhi(m, n) + n) >> l     for 0 <= n < 2^31,
// where the paper's halving step is folded into the shift because n + mulhi
// cannot overflow 32 bits for n < 2^31.  The host computes (m, l) once per
// call; the kernels divide with scalar or vector multiplies instead of the
// ~30-instruction generic sequence.  constexpr, so the same code serves the
// host (and its tests) and the device.
#pragma once

#include <stdint.h>

namespace wmk {

struct FastDiv {
    uint32_t mul;
    uint32_t shift;
};

// d in [1, 2^31).
constexpr FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    return FastDiv{uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1), l};
}

// floor(n / d) for n in [0, 2^31).
constexpr uint32_t fastdiv(uint32_t n, FastDiv f) {
    return (uint32_t(((uint64_t)n * f.mul) >> 32) + n) >> f.shift;
}

}  // namespace wmk
