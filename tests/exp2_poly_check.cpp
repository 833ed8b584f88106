// Exhaustive host check of the device polynomial exp2 (exp2_poly.h) against
// the C library's exp2 in double precision.  Prints one line per range:
//   <lo> <hi> <count> <max_rel_err> <argmax>
// and then integer-exactness and monotonicity verdicts.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <omp.h>
#include "exp2_poly.h"

template <int DEG>
static void scan(float lo, float hi) {
    uint32_t blo, bhi;
    // iterate over bit patterns of the same sign
    if (lo < 0 || (lo == 0 && std::signbit(lo))) {  // negative range: bits from -0 up to lo
        float a = -0.0f; memcpy(&blo, &a, 4); memcpy(&bhi, &lo, 4);
    } else {
        memcpy(&blo, &lo, 4); memcpy(&bhi, &hi, 4);
    }
    double worst = 0; float warg = 0; long long cnt = (long long)bhi - blo + 1;
#pragma omp parallel
    {
        double w = 0; float wa = 0;
#pragma omp for schedule(static)
        for (long long b = blo; b <= (long long)bhi; ++b) {
            uint32_t u = (uint32_t)b; float x; memcpy(&x, &u, 4);
            double ref = std::exp2((double)x);
            double got = (double)fa_exp2::exp2_poly<DEG>(x);
            double e = std::fabs(got / ref - 1.0);
            if (e > w) { w = e; wa = x; }
        }
#pragma omp critical
        { if (w > worst) { worst = w; warg = wa; } }
    }
    printf("deg%d %.9g %.9g %lld %.6e %.9g\n", DEG, lo, hi, cnt, worst, warg);
}

template <int DEG>
static void structure() {
    int exact = 1, mono = 1;
    for (int n = -126; n <= 8; ++n)
        if (fa_exp2::exp2_poly<DEG>((float)n) != std::ldexp(1.0f, n)) exact = 0;
    float prev = 0.0f;
    for (double x = -126.0; x <= 8.0; x += 1.0 / 4096) {
        float y = fa_exp2::exp2_poly<DEG>((float)x);
        if (y < prev) mono = 0;
        prev = y;
    }
    int zero = fa_exp2::exp2_poly<DEG>(-INFINITY) == 0.0f && fa_exp2::exp2_poly<DEG>(-126.5f) == 0.0f
               && fa_exp2::exp2_poly<DEG>(-1000.0f) == 0.0f;
    printf("deg%d exact_integers %d monotone %d zero_below %d\n", DEG, exact, mono, zero);
}

int main() {
    scan<3>(-126.0f, 0.0f);
    scan<3>(0.0f, 8.0f);
    structure<3>();
    scan<5>(-126.0f, 0.0f);
    scan<5>(0.0f, 8.0f);
    structure<5>();
    return 0;
}
