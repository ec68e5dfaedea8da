// Magic-number division shared by the planner and every kernel.
#pragma once

#include <cstdint>

namespace wgrad {

// Unsigned division by a runtime-constant divisor d >= 1, for dividends
// n < 2^31 (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, the round-up variant with a 32-bit multiplier):
//   l = ceil(log2 d), mul = floor(2^32 * (2^l - d) / d) + 1,
//   q = (mulhi(mul, n) + n) >> l.
// The (n, ho, wo) decode of the reduction index uses it so that the inner
// loop has no integer division.
struct MagicU32 {
    uint32_t mul;
    uint32_t shift;
};

inline MagicU32 make_magic(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return MagicU32{static_cast<uint32_t>(m), l};
}

inline uint32_t magic_div_host(uint32_t n, MagicU32 m) {
    uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(m.mul) * n) >> 32);
    return (t + n) >> m.shift;
}

}  // namespace wgrad
