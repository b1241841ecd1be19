// Offline weight preparation and the activation quantizer.
//
// The Q8_0 rule (llama.cpp-style blocks of 32 codes and an fp16 scale, used
// for weights and for int8 activations by emit_qwen38_generate, "Where the
// speed comes from") is implemented once, in common.hpp, and used here and
// in the GEMV prologue so that both produce the same bytes.
#include "common.hpp"
#include "internal.hpp"

namespace wsg {
namespace {

// Quantizes 32 floats (16-byte aligned) with the Q8_0 rule: codes to q[32],
// returns the scale bits.
__device__ inline uint16_t quantize_block32(const float* __restrict__ src, int8_t* q) {
    float v[32];
    const float4v* s4 = reinterpret_cast<const float4v*>(src);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4v t = s4[i];
        v[4 * i + 0] = t.x;
        v[4 * i + 1] = t.y;
        v[4 * i + 2] = t.z;
        v[4 * i + 3] = t.w;
    }
    return q8_quantize_block_bits(v, q);
}

// Block sizes are compile-time constants: reading blockDim.x is a vector load
// on this target, and every index computed from it would wait for that load.
constexpr int kActThreads = 64, kPrepThreads = 256;

__global__ void __launch_bounds__(kActThreads) quantize_act_kernel(const float* __restrict__ x, int nb,
                                                                   int8_t* __restrict__ q, uint16_t* __restrict__ d) {
    const int b = blockIdx.x * kActThreads + threadIdx.x;
    if (b >= nb) return;
    int8_t codes[32];
    const uint16_t d16 = quantize_block32(x + (int64_t)b * kBlock, codes);
    int4v* dst = reinterpret_cast<int4v*>(q + (int64_t)b * kBlock);
    int4v lo, hi;
    __builtin_memcpy(&lo, codes, 16);
    __builtin_memcpy(&hi, codes + 16, 16);
    dst[0] = lo;
    dst[1] = hi;
    d[b] = d16;
}

// Position of block b of a row inside the device layout.
struct BlockPos {
    int64_t scale, half_a, half_b;  // byte offsets from the row start
    int64_t pad_begin, pad_end;     // scale padding of the chunk (written by its last block)
    bool last_in_chunk;
};

__device__ inline BlockPos block_pos(int64_t b, int64_t k) {
    const int64_t C = chunk_count(k);
    const int64_t c = b / kChunkBlocks, j = b % kChunkBlocks;
    const int64_t nbc = (c == C - 1) ? last_chunk_blocks(k) : kChunkBlocks;
    const int64_t sb = scale_section_bytes(nbc);
    const int64_t base = c * kFullChunkBytes;
    BlockPos p;
    p.scale = base + 2 * j;
    p.half_a = base + sb + 16 * j;
    p.half_b = base + sb + 16 * nbc + 16 * j;
    p.pad_begin = base + 2 * nbc;
    p.pad_end = base + sb;
    p.last_in_chunk = (j == nbc - 1);
    return p;
}

__device__ inline void store_block(uint8_t* row, const BlockPos& p, uint16_t d16, const int8_t* codes) {
    *reinterpret_cast<uint16_t*>(row + p.scale) = d16;
    int4v lo, hi;
    __builtin_memcpy(&lo, codes, 16);
    __builtin_memcpy(&hi, codes + 16, 16);
    *reinterpret_cast<int4v*>(row + p.half_a) = lo;
    *reinterpret_cast<int4v*>(row + p.half_b) = hi;
    if (p.last_in_chunk)
        for (int64_t i = p.pad_begin; i < p.pad_end; ++i) row[i] = 0;
}

__global__ void quantize_weights_kernel(const float* __restrict__ w, int64_t n, int64_t k,
                                        uint8_t* __restrict__ out) {
    const int64_t nb = k / kBlock;
    const int64_t total = n * nb;
    const int64_t row_bytes = packed_row_bytes(k);
    const int64_t stride = (int64_t)gridDim.x * kPrepThreads;
    for (int64_t t = (int64_t)blockIdx.x * kPrepThreads + threadIdx.x; t < total; t += stride) {
        const int64_t r = t / nb, b = t % nb;
        int8_t codes[32];
        const uint16_t d16 = quantize_block32(w + r * k + b * kBlock, codes);
        store_block(out + r * row_bytes, block_pos(b, k), d16, codes);
    }
}

// 4-bit blocks (the W4 format): d16 = fp16(max|w| / 7), code = the fp32
// quotient w / d16 rounded half away from zero, clamped to [-7, 7], stored
// as code + 8 in the layout of q4_row_bytes; the thread of a row's last
// block also zeroes the padding of that chunk's scale section.
__global__ void quantize_q4_kernel(const float* __restrict__ w, int64_t n, int64_t k, uint8_t* __restrict__ out) {
    const int64_t nb = k / kBlock;
    const int64_t total = n * nb;
    const int64_t row_bytes = q4_row_bytes(k);
    const int64_t stride = (int64_t)gridDim.x * kPrepThreads;
    for (int64_t t = (int64_t)blockIdx.x * kPrepThreads + threadIdx.x; t < total; t += stride) {
        const int64_t r = t / nb, b = t % nb;
        const float* x = w + r * k + b * kBlock;
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < kBlock; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
        uint16_t d16 = float_to_half_bits_rne(amax / 7.0f);
        const float df = half_bits_to_float(d16);
        if (df == 0.0f) d16 = 0;
        uint8_t nib[kBlock];
#pragma unroll
        for (int i = 0; i < kBlock; ++i) {
            float c = df == 0.0f ? 0.0f : roundf(x[i] / df);
            c = c > 7.0f ? 7.0f : (c < -7.0f ? -7.0f : c);
            nib[i] = (uint8_t)((int)c + 8);
        }
        const int64_t c = b / kChunkBlocks, bb = b % kChunkBlocks;
        const int64_t nbc = c == chunk_count(k) - 1 ? last_chunk_blocks(k) : kChunkBlocks;
        const int64_t sb = scale_section_bytes(nbc);
        uint8_t* chunk = out + r * row_bytes + c * kFullChunkBytesQ4;
        chunk[2 * bb] = (uint8_t)(d16 & 0xFF);
        chunk[2 * bb + 1] = (uint8_t)(d16 >> 8);
#pragma unroll
        for (int j = 0; j < 16; ++j) chunk[sb + 16 * bb + j] = (uint8_t)(nib[j] | (nib[j + 16] << 4));
        if (bb == nbc - 1)
            for (int64_t p = 2 * nbc; p < sb; ++p) chunk[p] = 0;
    }
}

__global__ void pack_kernel(const uint8_t* __restrict__ aos, int64_t n, int64_t k, uint8_t* __restrict__ out) {
    const int64_t nb = k / kBlock;
    const int64_t total = n * nb;
    const int64_t row_bytes = packed_row_bytes(k);
    const int64_t stride = (int64_t)gridDim.x * kPrepThreads;
    for (int64_t t = (int64_t)blockIdx.x * kPrepThreads + threadIdx.x; t < total; t += stride) {
        const int64_t r = t / nb, b = t % nb;
        const uint8_t* src = aos + t * 34;
        const uint16_t d16 = (uint16_t)(src[0] | (src[1] << 8));
        int8_t codes[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) codes[i] = (int8_t)src[2 + i];
        store_block(out + r * row_bytes, block_pos(b, k), d16, codes);
    }
}

__global__ void convert_bf16_kernel(const float* __restrict__ in, int64_t count, uint16_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * kPrepThreads;
    for (int64_t i = (int64_t)blockIdx.x * kPrepThreads + threadIdx.x; i < count; i += stride) {
        const uint32_t b = __float_as_uint(in[i]);
        uint16_t r;
        if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) {
            r = (uint16_t)((b >> 16) | 0x0040u);  // quiet NaN, sign kept
        } else {
            // round to nearest even on the 16 dropped bits (carries into the
            // exponent give the correctly rounded neighbour, up to infinity)
            r = (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
        }
        out[i] = r;
    }
}

__global__ void fill_zero_kernel(float* __restrict__ y, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kPrepThreads;
    for (int64_t i = (int64_t)blockIdx.x * kPrepThreads + threadIdx.x; i < n; i += stride) y[i] = 0.0f;
}

unsigned grid_for(int64_t items, int block) {
    int64_t g = (items + block - 1) / block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (unsigned)g;
}

}  // namespace

int fill_zero_f32(float* y, int64_t n, hipStream_t stream) {
    if (n <= 0) return WSG_OK;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n, kPrepThreads)), dim3(kPrepThreads), 0, stream, y, n);
    return launch_status();
}

}  // namespace wsg

using namespace wsg;

extern "C" {

int64_t q8_0_row_bytes(int64_t k) {
    if (k <= 0 || k % kBlock) return 0;
    return packed_row_bytes(k);
}

int64_t q8_0_packed_bytes(int64_t n, int64_t k) {
    if (n <= 0 || k <= 0 || k % kBlock) return 0;
    return n * packed_row_bytes(k);
}

int64_t act_q8_0_bytes(int64_t k) {
    if (k <= 0 || k % kBlock) return 0;
    return k + k / 16;
}

int quantize_act_q8_0(const float* x, int64_t k, void* x_q8, hipStream_t stream) {
    if (k < 0 || k > kMaxDim || k % kBlock) return WSG_ERR_SHAPE;
    if (k == 0) return WSG_OK;
    if (!x || !x_q8) return WSG_ERR_NULL;
    if (!aligned(x, 16) || !aligned(x_q8, 16)) return WSG_ERR_ALIGN;
    const int nb = (int)(k / kBlock);
    int8_t* q = static_cast<int8_t*>(x_q8);
    uint16_t* d = reinterpret_cast<uint16_t*>(q + k);
    hipLaunchKernelGGL(quantize_act_kernel, dim3(grid_for(nb, kActThreads)), dim3(kActThreads), 0, stream, x, nb, q, d);
    return launch_status();
}

int quantize_q8_0_weights(const float* w, int64_t n, int64_t k, void* w_packed, hipStream_t stream) {
    if (n < 0 || k < 0 || n > kMaxDim || k > kMaxDim || k % kBlock) return WSG_ERR_SHAPE;
    if (n == 0 || k == 0) return WSG_OK;
    if (!w || !w_packed) return WSG_ERR_NULL;
    if (!aligned(w, 16) || !aligned(w_packed, 16)) return WSG_ERR_ALIGN;
    hipLaunchKernelGGL(quantize_weights_kernel, dim3(grid_for(n * (k / kBlock), kPrepThreads)), dim3(kPrepThreads), 0,
                       stream, w, n, k, static_cast<uint8_t*>(w_packed));
    return launch_status();
}

int64_t q4_0_row_bytes(int64_t k) {
    if (k < 0 || k > kMaxDim || k % kBlock) return -1;
    return q4_row_bytes(k);
}

int64_t q4_0_packed_bytes(int64_t n, int64_t k) {
    if (n < 0 || k < 0 || n > kMaxDim || k > kMaxDim || k % kBlock) return -1;
    return n * q4_row_bytes(k);
}

int quantize_q4_0_weights(const float* w, int64_t n, int64_t k, void* w_packed, hipStream_t stream) {
    if (n < 0 || k < 0 || n > kMaxDim || k > kMaxDim || k % kBlock) return WSG_ERR_SHAPE;
    if (n == 0 || k == 0) return WSG_OK;
    if (!w || !w_packed) return WSG_ERR_NULL;
    if (!aligned(w, 16) || !aligned(w_packed, 16)) return WSG_ERR_ALIGN;
    hipLaunchKernelGGL(quantize_q4_kernel, dim3(grid_for(n * (k / kBlock), kPrepThreads)), dim3(kPrepThreads), 0,
                       stream, w, n, k, static_cast<uint8_t*>(w_packed));
    return launch_status();
}

int pack_q8_0(const void* blocks_aos, int64_t n, int64_t k, void* w_packed, hipStream_t stream) {
    if (n < 0 || k < 0 || n > kMaxDim || k > kMaxDim || k % kBlock) return WSG_ERR_SHAPE;
    if (n == 0 || k == 0) return WSG_OK;
    if (!blocks_aos || !w_packed) return WSG_ERR_NULL;
    if (!aligned(w_packed, 16)) return WSG_ERR_ALIGN;
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for(n * (k / kBlock), kPrepThreads)), dim3(kPrepThreads), 0, stream,
                       static_cast<const uint8_t*>(blocks_aos), n, k, static_cast<uint8_t*>(w_packed));
    return launch_status();
}

int convert_bf16(const float* in, int64_t count, uint16_t* out, hipStream_t stream) {
    if (count < 0) return WSG_ERR_SHAPE;
    if (count == 0) return WSG_OK;
    if (!in || !out) return WSG_ERR_NULL;
    if (!aligned(in, 4) || !aligned(out, 2)) return WSG_ERR_ALIGN;
    hipLaunchKernelGGL(convert_bf16_kernel, dim3(grid_for(count, kPrepThreads)), dim3(kPrepThreads), 0, stream, in,
                       count, out);
    return launch_status();
}

}  // extern "C"
