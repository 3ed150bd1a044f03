// codec_math.hpp -- fp32 steps of the quantizer that the host-side tests
// check exhaustively, shared by the kernel and those tests.
#pragma once

#include <cmath>

#ifdef __HIPCC__
#define KIVI_CODEC_HD __host__ __device__
#else
#define KIVI_CODEC_HD
#endif

namespace kivi {

// x / y correctly rounded (IEEE fp32, round to nearest even) for y = 3 or 15,
// the 2^b - 1 of b = 2 and 4, without a division: q0 = x c with c = 1/y
// rounded, the residual x - y q0 (exact, by one fma), and q0 + r c (one more
// fma). The quantizer's x is the range of a group of fp16 values, a
// difference rounded to fp32: 0 or a value in [2^-24, 131008]. For every fp32
// x in [2^-24, 2^17] and for 0 this equals x / y (checked on the host for
// both divisors; an IEEE division takes about ten instructions on gfx950).
KIVI_CODEC_HD inline float div_by_levels(float x, float y, float c) {
    const float q0 = x * c;
    const float r = std::fma(-q0, y, x);
    return std::fma(r, c, q0);
}

}  // namespace kivi
