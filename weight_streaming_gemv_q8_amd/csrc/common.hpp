// Device helpers shared by the wsgemv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8rule.hpp"

namespace wsg {

constexpr int kWave = 64;
constexpr int kBlock = 32;             // Q8_0 block: 32 weights, one fp16 scale
constexpr int kChunkBlocks = 64;       // one block per lane of a wave
constexpr int kChunkWeights = kChunkBlocks * kBlock;  // 2048
constexpr int kFullChunkBytes = 2 * kChunkBlocks + kChunkWeights;  // 128 scale + 2048 code bytes

typedef int int4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- DPP moves
// Cross-lane moves within rows of 16 lanes (data-parallel primitives of the
// vector ALU): quad_perm [1,0,3,2] (lane ^ 1) and [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane 7 - i within 8), row_mirror (lane 15 - i within 16)
// and row_bcast:15 (lane 15 of each row into the next row, for the rows the
// row mask enables; the others keep `old`).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140,
              kDppRowBcast15 = 0x142;
template <int CTRL, int ROWS = 0xF>
__device__ inline float dpp_f32(float v, float old = 0.0f) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                   __builtin_bit_cast(int, v), CTRL, ROWS, 0xF,
                                                                   false));
}

// ------------------------------------------------------------- Q8_0 layout
// Bytes of a chunk's scale section: 2 bytes per block, padded to 16.
__host__ __device__ inline int64_t scale_section_bytes(int64_t nb) { return (2 * nb + 15) & ~int64_t(15); }

__host__ __device__ inline int64_t chunk_count(int64_t k) { return (k / kBlock + kChunkBlocks - 1) / kChunkBlocks; }

__host__ __device__ inline int64_t last_chunk_blocks(int64_t k) {
    const int64_t nb = k / kBlock;
    return nb - (chunk_count(k) - 1) * kChunkBlocks;
}

__host__ __device__ inline int64_t packed_row_bytes(int64_t k) {
    if (k <= 0) return 0;
    const int64_t c = chunk_count(k);
    const int64_t nl = last_chunk_blocks(k);
    return (c - 1) * kFullChunkBytes + scale_section_bytes(nl) + 32 * nl;
}

// ------------------------------------------------------------- W4 layout
// 4-bit blocks: per 2048-weight chunk [64 fp16 scales][64 x 16 code bytes]
// (a block's byte j: code j in the low nibble, code j + 16 in the high one,
// codes stored as q + 8); the last chunk's scale section padded to 16.
constexpr int kFullChunkBytesQ4 = 2 * kChunkBlocks + kChunkWeights / 2;  // 128 + 1024

__host__ __device__ inline int64_t q4_row_bytes(int64_t k) {
    if (k <= 0) return 0;
    const int64_t c = chunk_count(k);
    const int64_t nl = last_chunk_blocks(k);
    return (c - 1) * kFullChunkBytesQ4 + scale_section_bytes(nl) + 16 * nl;
}

// --------------------------------------------------------------- loads
// Weight stream loads: 16 bytes per lane, optionally marked non-temporal so
// the stream does not evict the (re-used) activation from L2.
// A pointer known to address global memory: loads through it compile to
// global_* instructions even when the pointer itself was read from memory.
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;

template <bool NT>
__device__ inline int4v load16(gptr<void> p) {
    if constexpr (NT) {
        return __builtin_nontemporal_load(reinterpret_cast<gptr<int4v>>(p));
    } else {
        return *reinterpret_cast<gptr<int4v>>(p);
    }
}

template <bool NT>
__device__ inline uint16_t load_u16(gptr<void> p) {
    if constexpr (NT) {
        return __builtin_nontemporal_load(reinterpret_cast<gptr<uint16_t>>(p));
    } else {
        return *reinterpret_cast<gptr<uint16_t>>(p);
    }
}

template <bool NT>
__device__ inline int4v load16(const void* p) {
    if constexpr (NT) {
        return __builtin_nontemporal_load(reinterpret_cast<const int4v*>(p));
    } else {
        return *reinterpret_cast<const int4v*>(p);
    }
}

template <bool NT>
__device__ inline uint16_t load_u16(const void* p) {
    if constexpr (NT) {
        return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
    } else {
        return *reinterpret_cast<const uint16_t*>(p);
    }
}

__device__ inline float half_bits_to_float(uint16_t h) {
    _Float16 f;
    __builtin_memcpy(&f, &h, 2);
    return (float)f;
}

__device__ inline uint16_t float_to_half_bits_rne(float x) {
    _Float16 f = (_Float16)x;  // v_cvt_f16_f32: round to nearest even
    uint16_t h;
    __builtin_memcpy(&h, &f, 2);
    return h;
}

// ------------------------------------------------------ Q8_0 block quantizer
// The Q8_0 rule for one 32-value block, in fp32 as the oracle takes it:
// d = fp16_RNE(max|v| / 127) (IEEE divide), q_i = clamp(round half away from
// zero of v_i / float(d), -127, 127) (IEEE divide by the stored scale,
// decided without a per-value divide by q8_code_exact); a zero scale stores
// d = +0 and q = 0.  Returns the scale bits.
__device__ inline uint16_t q8_scale_bits(float amax) { return float_to_half_bits_rne(amax / 127.0f); }

__device__ inline uint16_t q8_quantize_block_bits(const float* v, int8_t* q) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    const uint16_t d16 = q8_scale_bits(amax);
    const float d = half_bits_to_float(d16);
    if (d == 0.0f) {
#pragma unroll
        for (int i = 0; i < 32; ++i) q[i] = 0;
        return 0;
    }
    const float r = 1.0f / d;
#pragma unroll
    for (int i = 0; i < 32; ++i) q[i] = (int8_t)q8_code_exact(v[i], d, r);
    return d16;
}

// The same rule for a block spread over a quad: four consecutive lanes (all
// active together) hold the block's 32 values, eight each, in order.  The
// block maximum meets in a quad reduction, every lane derives the same
// scale and packs its eight codes little-endian into lo (values 0-3) and hi
// (values 4-7).  Returns the scale bits.
__device__ inline uint16_t q8_quad_codes(const float (&v)[8], uint32_t& lo, uint32_t& hi) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    amax = __builtin_fmaxf(amax, dpp_f32<kDppXor1>(amax));
    amax = __builtin_fmaxf(amax, dpp_f32<kDppXor2>(amax));
    const uint16_t d16 = q8_scale_bits(amax);
    const float d = half_bits_to_float(d16);
    lo = 0;
    hi = 0;
    if (d != 0.0f) {
        const float r = 1.0f / d;
        int q[8];
        bool any_near = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            bool near;
            q[i] = q8_code_fast(v[i], r, near);
            any_near |= near;
        }
        if (__any(any_near)) {  // rare: a value within 4e-5 of a rounding boundary
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = q8_code(v[i], d, r);
        }
        lo = (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) | ((uint32_t)(q[2] & 0xFF) << 16) |
             ((uint32_t)q[3] << 24);
        hi = (uint32_t)(q[4] & 0xFF) | ((uint32_t)(q[5] & 0xFF) << 8) | ((uint32_t)(q[6] & 0xFF) << 16) |
             ((uint32_t)q[7] << 24);
    }
    return d16;
}

// The wave's index in its workgroup, as a wave-uniform (scalar) value: the
// compiler cannot tell that threadIdx.x / 64 is the same in every lane, and
// without this everything derived from it (rows, chunk addresses, loop
// bounds) would be computed per lane in vector registers.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)); }

// ------------------------------------------------------- wave reductions
// A sum over the 64 lanes of a wave as a fixed binary tree: lanes pair up
// with lane ^ 1, then quads with their neighbour quad (every lane of a quad
// holds the same value by then), then 8-lane groups, all as DPP moves within
// rows of 16 lanes (no LDS round trip); lane 15 of rows 0 and 2 is added
// into rows 1 and 3, and the result is row sums (0 + 1) + (2 + 3), read from
// lanes 31 and 63 into a wave-uniform value.  The order of additions does
// not depend on the data or on which row is reduced.
__device__ inline float wave_sum(float v) {
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    v += dpp_f32<kDppMirror>(v);
    v += dpp_f32<kDppRowBcast15, 0xA>(v);
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    return lo + hi;
}

__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t u = __shfl_xor(v, o, kWave);
        v = u > v ? u : v;
    }
    return v;
}

// --------------------------------------------------------- argmax keys
// Order-preserving 64-bit key for (value, index): larger value wins; among
// IEEE-equal values (-0 == +0 after canonicalization) the lower index wins.
__device__ inline uint64_t argmax_key(float v, uint32_t idx) {
    if (v == 0.0f) v = 0.0f;  // -0 -> +0
    const uint32_t b = __float_as_uint(v);
    const uint32_t ordered = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)ordered << 32) | (uint64_t)(~idx);
}

__device__ inline uint32_t argmax_key_index(uint64_t key) { return ~(uint32_t)(key & 0xFFFFFFFFu); }

}  // namespace wsg
