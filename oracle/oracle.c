/* CPU ORACLE for the batch-1 decode GEMV weight stream -- TEST
 * INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the bench may load this library; the product path never
 * does.  It shares no code, header, table or helper with the HIP library.
 *
 * Plain, slow, obviously correct: fp64 arithmetic (every product below is
 * exact in fp64, so the only rounding is the running sum), no blocking, no
 * SIMD, single thread.  Where the pages fix a precision the oracle uses it:
 * the Q8_0 quantizer takes its decisions in fp32, as the kernel does.
 *
 * What it computes (the pages: emit_qwen38_generate, "Where the speed comes
 * from"; qwen3-8b-rtx4080-cutedsl, "Decode GEMV path"; GPU Kernel Lab,
 * "Decode integration"):
 *   y = W.x for a row-major W, one activation vector, batch 1;
 *   W in BF16, or in Q8_0 blocks (32 int8 codes + one fp16 scale per 32
 *   consecutive weights of a row, as in llama.cpp);
 *   x either quantized to int8 per 32-block with the same Q8_0 rule (the
 *   int8-dot form, deq mode 0) or kept in f32 (the dequantizing form,
 *   deq modes 1/2, "removes the activation quantization error");
 *   the LM head ends with an argmax whose ties go to the lowest index.
 *
 * Readings where the pages are silent (listed with reasons in the design
 * notes):
 *   - scale d = fp16_RNE(max|x| / 127) with the divide done in IEEE fp32;
 *     codes q = clamp(round_half_away(x / d16), -127, 127) against the
 *     STORED fp16 scale, fp32 divide;
 *   - a block whose fp16 scale is zero stores d = +0 and q = 0;
 *   - activation blocks use the same rule and an fp16 scale;
 *   - argmax ties (IEEE equality, so -0 == +0) resolve to the lowest index.
 *
 * Parity of every function here is pinned by tests against library
 * routines, closed forms, invariants and brute force (see tests/).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ O1 --
 * IEEE-754 binary16 and bfloat16 codecs, round-to-nearest-even, subnormals
 * handled.  Written from the format definitions:
 *   binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; normal
 *             values (1.f) * 2^(e-15), subnormals (0.f) * 2^-14;
 *   bfloat16: the top 16 bits of a binary32 (1 sign, 8 exponent bias 127,
 *             7 fraction bits).
 */

static uint32_t f32_bits(float x) {
    uint32_t b;
    memcpy(&b, &x, 4);
    return b;
}

/* Round the exact value m * 2^e (m < 2^25) to an integer multiple of 2^qe,
 * nearest, ties to even; returns the multiple count. */
static uint64_t round_to_quantum(uint64_t m, int e, int qe) {
    int shift = qe - e;
    if (shift <= 0) return m << (-shift);
    if (shift > 40) return 0;
    uint64_t q = m >> shift;
    uint64_t rem = m & ((1ull << shift) - 1);
    uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) q += 1;
    return q;
}

/* Decompose a finite nonzero binary32 into m * 2^e with m an integer. */
static void f32_decompose(uint32_t a, uint64_t* m, int* e) {
    uint32_t ex = (a >> 23) & 0xFF, fr = a & 0x7FFFFF;
    if (ex == 0) {
        *m = fr;
        *e = 1 - 127 - 23;
    } else {
        *m = fr | 0x800000u;
        *e = (int)ex - 127 - 23;
    }
}

/* floor(log2(m * 2^e)) for m > 0 */
static int ilog2_value(uint64_t m, int e) {
    int l = 63;
    while (!((m >> l) & 1)) --l;
    return l + e;
}

uint16_t orc_f32_to_f16(float x) {
    uint32_t b = f32_bits(x);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
    uint32_t a = b & 0x7FFFFFFFu;
    if (a >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (a > 0x7F800000u ? 0x200u : 0u));
    if (a == 0) return sign;
    uint64_t m;
    int e;
    f32_decompose(a, &m, &e);
    int lg = ilog2_value(m, e);
    if (lg < -14) {
        /* subnormal range: quantum 2^-24; a count of 1024 is the smallest
         * normal, whose encoding is the same integer */
        uint64_t q = round_to_quantum(m, e, -24);
        return (uint16_t)(sign | (uint16_t)q);
    }
    uint64_t q = round_to_quantum(m, e, lg - 10); /* in [1024, 2048] */
    int be = lg + 15;
    if (q == 2048) {
        q = 1024;
        be += 1;
    }
    if (be >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)(be << 10) | (uint16_t)(q - 1024));
}

double orc_f16_to_f64(uint16_t h) {
    int s = (h >> 15) & 1, ex = (h >> 10) & 0x1F, fr = h & 0x3FF;
    double v;
    if (ex == 0x1F) v = fr ? NAN : INFINITY;
    else if (ex == 0) v = ldexp((double)fr, -24);
    else v = ldexp((double)(fr + 1024), ex - 25);
    return s ? -v : v;
}

uint16_t orc_f32_to_bf16(float x) {
    uint32_t b = f32_bits(x);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
    uint32_t a = b & 0x7FFFFFFFu;
    if (a >= 0x7F800000u) return (uint16_t)(sign | 0x7F80u | (a > 0x7F800000u ? 0x40u : 0u));
    if (a == 0) return sign;
    uint64_t m;
    int e;
    f32_decompose(a, &m, &e);
    int lg = ilog2_value(m, e);
    if (lg < -126) {
        /* binary32 subnormal range: bfloat16 quantum 2^-133 */
        uint64_t q = round_to_quantum(m, e, -133);
        return (uint16_t)(sign | (uint16_t)q);
    }
    uint64_t q = round_to_quantum(m, e, lg - 7); /* in [128, 256] */
    int be = lg + 127;
    if (q == 256) {
        q = 128;
        be += 1;
    }
    if (be >= 255) return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | (uint16_t)(be << 7) | (uint16_t)(q - 128));
}

double orc_bf16_to_f64(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
}

/* Element-wise array forms of the two encoders and decoders. */
int orc_q8_code(float v, uint16_t d16);
void orc_q8_code_array(const float* v, const uint16_t* d16, int64_t n, int8_t* out);

void orc_f32_to_f16_array(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f64_array(const uint16_t* h, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f64(h[i]);
}

void orc_f32_to_bf16_array(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(x[i]);
}

void orc_bf16_to_f64_array(const uint16_t* h, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f64(h[i]);
}

/* ------------------------------------------------------------------ O2 --
 * One Q8_0 code: the fp32 quotient v / d (IEEE divide by the stored fp16
 * scale), rounded half away from zero, clamped to [-127, 127].  d16 must be
 * a positive finite fp16 value. */
int orc_q8_code(float v, uint16_t d16) {
    float df = (float)orc_f16_to_f64(d16); /* exact */
    float r = roundf(v / df);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int)r;
}

void orc_q8_code_array(const float* v, const uint16_t* d16, int64_t n, int8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (int8_t)orc_q8_code(v[i], d16[i]);
}

/* Q8_0 block quantizer, for weights (offline) and activations (per call).
 * rows x k floats, k % 32 == 0; writes d[rows][k/32] (fp16 bits) and
 * q[rows][k].  Returns 0, or -1 on a bad shape, -2 on a non-finite input
 * or an fp16 scale overflow (both outside the contract).
 */
int orc_quantize_q8_0(const float* x, int64_t rows, int64_t k, uint16_t* d, int8_t* q) {
    if (rows < 0 || k < 0 || k % 32 != 0) return -1;
    const int64_t nb = k / 32;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* xb = x + r * k + b * 32;
            int8_t* qb = q + r * k + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                if (!isfinite(xb[i])) return -2;
                float a = fabsf(xb[i]);
                if (a > amax) amax = a;
            }
            float dd = amax / 127.0f; /* IEEE fp32 divide */
            uint16_t d16 = orc_f32_to_f16(dd);
            if ((d16 & 0x7C00u) == 0x7C00u) return -2;
            float df = (float)orc_f16_to_f64(d16); /* exact */
            if (df == 0.0f) {
                d[r * nb + b] = 0;
                for (int i = 0; i < 32; ++i) qb[i] = 0;
                continue;
            }
            d[r * nb + b] = d16;
            for (int i = 0; i < 32; ++i) qb[i] = (int8_t)orc_q8_code(xb[i], d16);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ O3 --
 * Q8_0 weights x int8 activations (deq mode 0).  For row r and block b:
 *   s[r,b] = sum_i qw[r,32b+i] * qx[32b+i]               (exact integer)
 *   y[r]   = sum_b d_w[r,b] * d_x[b] * s[r,b]            (fp64; each term
 *            exact: 11 + 11 + 20 significant bits)
 *   den[r] = sum_b |d_w[r,b] * d_x[b] * s[r,b]|          (tolerance scale)
 * dots (nullable) receives s as int32[n][k/32].  Returns 0, -1 bad shape,
 * -3 if a block dot does not fit int32 (cannot happen for codes in
 * [-128, 127]: |s| <= 32*128*128).
 */
int orc_gemv_q8_act_q8(const uint16_t* dw, const int8_t* qw, int64_t n, int64_t k,
                       const uint16_t* dx, const int8_t* qx, double* y, double* den,
                       int32_t* dots) {
    if (n < 0 || k < 0 || k % 32 != 0) return -1;
    const int64_t nb = k / 32;
    for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0, mag = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            int64_t s = 0;
            for (int i = 0; i < 32; ++i)
                s += (int64_t)qw[r * k + b * 32 + i] * (int64_t)qx[b * 32 + i];
            if (s > INT32_MAX || s < INT32_MIN) return -3;
            if (dots) dots[r * nb + b] = (int32_t)s;
            double t = orc_f16_to_f64(dw[r * nb + b]) * orc_f16_to_f64(dx[b]) * (double)s;
            acc += t;
            mag += fabs(t);
        }
        y[r] = acc;
        if (den) den[r] = mag;
    }
    return 0;
}

/* ------------------------------------------------------------------ O4 --
 * Q8_0 weights x f32 activations (the dequantizing form, deq modes 1/2):
 *   y[r]   = sum_b sum_i d_w[r,b] * qw[r,32b+i] * x[32b+i]
 *   den[r] = sum_b sum_i |d_w[r,b] * qw[r,32b+i] * x[32b+i]|
 * Each term is exact in fp64 (11 + 8 + 24 significant bits).
 */
int orc_gemv_q8_act_f32(const uint16_t* dw, const int8_t* qw, int64_t n, int64_t k,
                        const float* x, double* y, double* den) {
    if (n < 0 || k < 0 || k % 32 != 0) return -1;
    const int64_t nb = k / 32;
    for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0, mag = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            double dwb = orc_f16_to_f64(dw[r * nb + b]);
            for (int i = 0; i < 32; ++i) {
                double t = dwb * (double)qw[r * k + b * 32 + i] * (double)x[b * 32 + i];
                acc += t;
                mag += fabs(t);
            }
        }
        y[r] = acc;
        if (den) den[r] = mag;
    }
    return 0;
}

/* ------------------------------------------------------------------ O5 --
 * BF16 weights x f32 activations:
 *   y[r] = sum_i bf16(w[r,i]) * x[i],  den[r] = sum_i |bf16(w[r,i]) * x[i]|
 * Each term is exact in fp64 (8 + 24 significant bits).
 */
int orc_gemv_bf16(const uint16_t* w, int64_t n, int64_t k, const float* x, double* y,
                  double* den) {
    if (n < 0 || k < 0) return -1;
    for (int64_t r = 0; r < n; ++r) {
        double acc = 0.0, mag = 0.0;
        for (int64_t i = 0; i < k; ++i) {
            double t = orc_bf16_to_f64(w[r * k + i]) * (double)x[i];
            acc += t;
            mag += fabs(t);
        }
        y[r] = acc;
        if (den) den[r] = mag;
    }
    return 0;
}

/* ------------------------------------------------------------------ O6 --
 * argmax: the smallest index i with v[i] == max(v) under IEEE equality
 * (so -0.0 and +0.0 tie).  Returns -1 for n <= 0 or if any NaN is present
 * (outside the contract).
 */
int64_t orc_argmax_f64(const double* v, int64_t n) {
    if (n <= 0) return -1;
    for (int64_t i = 0; i < n; ++i)
        if (isnan(v[i])) return -1;
    double best = v[0];
    for (int64_t i = 1; i < n; ++i)
        if (v[i] > best) best = v[i];
    for (int64_t i = 0; i < n; ++i)
        if (v[i] == best) return i;
    return -1;
}

int64_t orc_argmax_f32(const float* v, int64_t n) {
    if (n <= 0) return -1;
    for (int64_t i = 0; i < n; ++i)
        if (isnan(v[i])) return -1;
    float best = v[0];
    for (int64_t i = 1; i < n; ++i)
        if (v[i] > best) best = v[i];
    for (int64_t i = 0; i < n; ++i)
        if (v[i] == best) return i;
    return -1;
}

/* ------------------------------------------------------------------ O9 --
 * The step either side of every GEMV: the residual add, the next RMSNorm
 * and the activation re-quantization (emit_qwen38_generate, "Where the
 * speed comes from", item 3, does the three in one kernel; GPU Kernel Lab,
 * "Decode integration": RMSNorm with an FP32 reduction and residual
 * fusion).  The pages give no formula; the readings (listed in the design
 * notes) are
 *   h'  = h + r, rounded once to fp32 (the residual stream after the add;
 *         r may be absent: h' = h);
 *   y_i = h'_i / sqrt(mean_j h'_j^2 + eps) * g_i, with eps and the
 *         per-channel weight g given by the caller;
 * and y is then quantized by the Q8_0 rule above (orc_quantize_q8_0 on the
 * fp32 values the kernel produced).  Here the add is one IEEE fp32 rounding
 * (exact in fp64, then rounded), the squares are exact in fp64, and the
 * mean, the square root and the products are fp64.
 */
void orc_residual_rmsnorm(const float* h, const float* r, const float* g, int64_t k, double eps, float* h_out,
                          double* y_out) {
    double ss = 0.0;
    for (int64_t i = 0; i < k; ++i) {
        const float a = r ? (float)((double)h[i] + (double)r[i]) : h[i];
        h_out[i] = a;
        ss += (double)a * (double)a;
    }
    const double s = 1.0 / sqrt(ss / (double)k + eps);
    for (int64_t i = 0; i < k; ++i) y_out[i] = (double)h_out[i] * s * (double)g[i];
}

/* O10: the SwiGLU epilogue of the gate+up GEMV (GPU Kernel Lab, "What we
 * built", "Decode integration", "Quantization experiments": a dual gate/up
 * projection fused with SwiGLU at batch 1).  The pages give no formula; the
 * reading (listed in the design notes) is the standard gated activation of
 * the MLP, y_i = silu(g_i) * u_i with silu(x) = x / (1 + exp(-x)), where g
 * is the gate half and u the up half of the concatenated gate+up output
 * (gate rows first).  All fp64; exp(-x) overflowing to +inf for very
 * negative x gives silu(x) = -0, the limit. */
void orc_swiglu(const double* g, const double* u, int64_t n, double* y) {
    for (int64_t i = 0; i < n; ++i) {
        const double x = g[i];
        y[i] = x / (1.0 + exp(-x)) * u[i];
    }
}

/* O11: 4-bit weight blocks for the W4 GEMV (qwen3-8b-rtx4080-cutedsl,
 * "W4A16 dequant-fused GEMM": group-wise 4-bit weights at ~4.6 GB for the
 * 8B model; GPU Kernel Lab, "Quantization experiments").  The pages give
 * no 4-bit rule; the reading (listed in the design notes) is the Q8_0 rule
 * with 7 in place of 127: per block of 32, d = max|x| / 7 in IEEE fp32,
 * d16 = fp16(d), q = the fp32 quotient x / d16 rounded half away from zero,
 * clamped to [-7, 7]; an all-zero (or underflowing) block has d16 = +0 and
 * q = 0.  The stored block is 18 bytes (fp16 d and 16 bytes of 4-bit codes
 * q + 8), so y = sum_b d_w d_x s with s = sum_i q_w q_x is the int8 GEMV of
 * O3 with these codes. */
int orc_quantize_q4_0(const float* x, int64_t rows, int64_t k, uint16_t* d, int8_t* q) {
    if (rows < 0 || k < 0 || k % 32 != 0) return -1;
    const int64_t nb = k / 32;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* xb = x + r * k + b * 32;
            int8_t* qb = q + r * k + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                if (!isfinite(xb[i])) return -2;
                const float a = fabsf(xb[i]);
                if (a > amax) amax = a;
            }
            const uint16_t d16 = orc_f32_to_f16(amax / 7.0f);
            if ((d16 & 0x7C00u) == 0x7C00u) return -2;
            const float df = (float)orc_f16_to_f64(d16);
            d[r * nb + b] = df == 0.0f ? 0 : d16;
            for (int i = 0; i < 32; ++i) {
                float c = df == 0.0f ? 0.0f : roundf(xb[i] / df);
                if (c > 7.0f) c = 7.0f;
                if (c < -7.0f) c = -7.0f;
                qb[i] = (int8_t)c;
            }
        }
    }
    return 0;
}
