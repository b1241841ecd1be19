/* Seeded, counter-based synthetic inputs for the batch-1 decode GEMV weight
 * stream.  This module is shared by the CPU oracle side and the GPU side of
 * every test and of the bench; it holds no arithmetic of the method itself
 * (no quantization, no dot products, no reductions): only random numbers
 * and their placement.
 *
 * Definition (identical in synth.c and synth_dev.hip; both are written from
 * this text):
 *
 *   mix64(z)   : the SplitMix64 output function (Steele, Lea, Flood,
 *                "Fast splittable pseudorandom number generators", 2014):
 *                z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *                z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31.
 *   word(key,n): the n-th output of a SplitMix64 generator whose state
 *                starts at key, i.e. mix64(key + (n+1)*0x9E3779B97F4A7C15)
 *                (arithmetic mod 2^64).
 *   key(seed,t): word(seed, t)   -- one independent stream per tensor id t.
 *
 *   normal(key, e, sigma): words 4e..4e+3 each give three 20-bit fields
 *                (bits 0-19, 20-39, 40-59); S = sum of the 12 fields;
 *                z = S - 6*(2^20-1), an integer with |z| < 2^23, converted
 *                to float exactly; value = z * (sigma * 2^-20) as ONE fp32
 *                multiply (Irwin-Hall(12): mean 0, variance ~1 after the
 *                2^-20 scaling).
 *   int8 q    : word(key, e) mod 255 - 127, in [-127, 127].
 *   fp16 scale: w = word(key, e): biased exponent 3 + (w >> 32) mod 4,
 *                mantissa w & 0x3FF, sign +: a positive normal fp16 in
 *                [2^-12, 2^-8), the range of Q8_0 scales of ~N(0,0.02)
 *                weights.
 */
#ifndef SYNTH_H
#define SYNTH_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

uint64_t synth_mix64(uint64_t z);
uint64_t synth_word(uint64_t key, uint64_t n);
uint64_t synth_key(uint64_t seed, uint64_t tensor);

/* out[i] = normal(key(seed,tensor), first + i, sigma) for i < count.
 * Multi-threaded over i; the bytes do not depend on the thread count. */
void synth_normal_f32(uint64_t seed, uint64_t tensor, int64_t first, int64_t count,
                      float sigma, float* out, int threads);

/* Rows of a row-major n x k matrix of normals (tensor id t): for each listed
 * row r, out[j*k + c] = normal(key, r*k + c, sigma). */
void synth_normal_rows_f32(uint64_t seed, uint64_t tensor, int64_t k, const int64_t* rows,
                           int64_t n_rows, float sigma, float* out, int threads);

/* out[i] = int8 draw at element first+i. */
void synth_int8(uint64_t seed, uint64_t tensor, int64_t first, int64_t count, int8_t* out);

/* out[i] = fp16 scale bits drawn at element first+i. */
void synth_f16_scale(uint64_t seed, uint64_t tensor, int64_t first, int64_t count, uint16_t* out);

/* Seeded partial Fisher-Yates over [0, n): writes the first m entries of the
 * shuffled permutation.  Draw i uses word(key(seed,tensor), i) mod (n - i). */
void synth_choose(uint64_t seed, uint64_t tensor, int64_t n, int64_t m, int64_t* out);

#ifdef __cplusplus
}
#endif
#endif
