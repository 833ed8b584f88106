// exp2_poly.h -- 2^x from FMAs, the software exponential of the hybrid split.
//
// The FlashAttention-4 explainer (gist.science, technical summary,
// methodology item 2) moves part of the softmax exponentials off the special
// function unit onto the FMA pipes as a degree 3 or 5 polynomial, accurate
// enough for bf16.  Method (Cody-Waite style range reduction, Horner
// evaluation, exponent scaling):
//
//   x <- max(x, -127);  n = floor(x);  f = x - n in [0, 1)
//   2^x = 2^n * p(f),  p(f) = 1 + c1 f + ... + cD f^D
//
// p(0) = 1 exactly, so integer x gives exact powers of two.  c1..cD minimise
// the maximum relative error of p(f) / 2^f on [0, 1]; they are printed by
// fit_exp2_poly.py next to this file (linear-programming minimax fit):
// 8.6e-5 for degree 3 and 9.2e-8 for degree 5 in exact arithmetic, a few
// fp32 ulp more once evaluated in fp32.  For x < -126 the result is 0
// (masked scores arrive as -inf and must give exactly 0).
//
// The header is plain C++ usable from host and device code; the host copy
// is what the exhaustive CPU test over [-126, 0] exercises.
#pragma once

#if defined(__HIPCC__)
#define FA_HD __host__ __device__ inline __attribute__((always_inline))
#else
#define FA_HD inline
#endif

#include <math.h>

namespace fa_exp2 {

constexpr float kD3C1 = 0.69511664f;
constexpr float kD3C2 = 0.22764498f;
constexpr float kD3C3 = 0.07706724f;

constexpr float kD5C1 = 0.69315106f;
constexpr float kD5C2 = 0.2401666f;
constexpr float kD5C3 = 0.055794485f;
constexpr float kD5C4 = 0.009022698f;
constexpr float kD5C5 = 0.0018650338f;

template <int DEG>
FA_HD float poly(float f) {
    if constexpr (DEG == 3) {
        return fmaf(fmaf(fmaf(kD3C3, f, kD3C2), f, kD3C1), f, 1.0f);
    } else {
        static_assert(DEG == 5, "degree 3 or 5");
        return fmaf(fmaf(fmaf(fmaf(fmaf(kD5C5, f, kD5C4), f, kD5C3), f, kD5C2), f, kD5C1), f, 1.0f);
    }
}

template <int DEG>
FA_HD float exp2_poly(float x) {
    float xc = fmaxf(x, -127.0f);
    float n = floorf(xc);
    float f = xc - n;
    float r = ldexpf(poly<DEG>(f), (int)n);
    return xc < -126.0f ? 0.0f : r;
}

}  // namespace fa_exp2
