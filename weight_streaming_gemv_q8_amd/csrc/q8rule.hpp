// The Q8_0 code of one value, decided exactly as
//     q = clamp(round_half_away(fl32(v / d)), -127, 127)
// (an IEEE fp32 divide by the stored fp16 scale d, then rounding half away
// from zero) but without a divide per value: the quotient is approximated
// by t = v * fl32(1/d), which is within |v/d| * 2^-23 of v/d, and only when
// t lies within 4e-5 of a rounding boundary b = m + 1/2 is the decision
// taken exactly:
//   fl32(v/d) >= b  <=>  v/d >= b - h_b  <=>  |v| >= (b - h_b) * d,
// where h_b is half the spacing of floats just below b (b has at most nine
// significant bits, so ties between b and its predecessor round to b).  The
// right-hand side has at most 36 significant bits and is exact in fp64.
// Written for both host and device so that the host test can check it
// against the oracle's plain divide on billions of values.
#pragma once

#include <stdint.h>

#ifndef __HIPCC__
#ifndef __host__
#define __host__
#endif
#ifndef __device__
#define __device__
#endif
#endif

namespace wsg {

__host__ __device__ inline int q8_code_exact(float v, float d, float r) {
    // d > 0 is an fp16 value; r = fl32(1 / d).
    const float a = __builtin_fabsf(v);
    const float ta = a * r;
    const float fl = __builtin_floorf(ta);
    const float b = fl + 0.5f;  // nearest boundary of the form m + 1/2
    int m;
    if (__builtin_fabsf(ta - b) < 4e-5f && ta < 256.0f) {
        // h_b: b = 0.5 sits on a binade edge (floats below are 2^-25 apart);
        // otherwise b in [2^e, 2^(e+1)) with floats 2^(e-23) apart
        double h;
        if (b == 0.5f) {
            h = 1.0 / 67108864.0;  // 2^-26
        } else {
            int e = 0;
            for (float p = 2.0f; p <= b; p *= 2.0f) ++e;
            h = 1.0;
            for (int i = 0; i < 24 - e; ++i) h *= 0.5;  // 2^(e-24), exact
        }
        const bool up = (double)a >= ((double)b - h) * (double)d;
        m = (int)fl + (up ? 1 : 0);
    } else {
        const float frac = ta - fl;  // exact
        m = (int)fl + (frac >= 0.5f ? 1 : 0);
    }
    if (m > 127) m = 127;
    return v < 0.0f ? -m : m;
}

// Branch-free form of the same rule for the common case: u = |v| r + 1/2 (one
// fused multiply-add, so no compiler contraction can change it) and
// m = floor(u), which equals the rule's code whenever u is at least 4e-5
// away from an integer (then |v/d| is at least ~4e-5 - 2^-23 away from the
// boundary m + 1/2, farther than the error of v r).  Otherwise `near` is set
// and the caller decides the code with q8_code_exact.  The fraction of u is
// exact (u - floor(u)), so is its distance to 1/2, and near is |fr - 1/2|
// above 1/2 - 4e-5.  The signed code is the truncation of u carrying v's
// sign (u >= 1/2, so that is sign(v) floor(u)), clamped to [-127, 127]:
// codes at and above the boundary 127.5 clamp to 127 either way, so they
// never need the exact test.  About seven vector instructions per value.
__host__ __device__ inline int q8_code_fast(float v, float r, bool& near) {
    const float u = __builtin_fmaf(__builtin_fabsf(v), r, 0.5f);
    const float fr = u - __builtin_floorf(u);  // exact
    near = __builtin_fabsf(fr - 0.5f) > 0.5f - 4e-5f;
    const int q = (int)__builtin_copysignf(u, v);
    return q > 127 ? 127 : (q < -127 ? -127 : q);
}

// The rule as the kernels apply it: the fast form, and the exact decision
// for values next to a boundary.
__host__ __device__ inline int q8_code(float v, float d, float r) {
    bool near;
    const int q = q8_code_fast(v, r, near);
    return near ? q8_code_exact(v, d, r) : q;
}

}  // namespace wsg
