// Host build of the HIP library's divide-free Q8_0 code rule, for the test
// that compares it with the oracle's plain IEEE divide on many values.
#include <math.h>
#include <stdint.h>

#include "q8rule.hpp"

static float f16_value(uint16_t h) {
    int ex = (h >> 10) & 0x1F, fr = h & 0x3FF;
    double v = ex == 0 ? ldexp((double)fr, -24) : ldexp((double)(fr + 1024), ex - 25);
    return (float)v;  // exact
}

extern "C" void fast_codes(const float* v, const uint16_t* d16, int64_t n, int8_t* out) {
    for (int64_t i = 0; i < n; ++i) {
        const float d = f16_value(d16[i]);
        const float r = 1.0f / d;
        out[i] = (int8_t)wsg::q8_code_exact(v[i], d, r);
    }
}

extern "C" void fast_split_codes(const float* v, const uint16_t* d16, int64_t n, int8_t* out) {
    for (int64_t i = 0; i < n; ++i) {
        const float d = f16_value(d16[i]);
        const float r = 1.0f / d;
        out[i] = (int8_t)wsg::q8_code(v[i], d, r);
    }
}
