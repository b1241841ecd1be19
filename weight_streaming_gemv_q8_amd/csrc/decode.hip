// The two calls that close the decode loop on the device (GPU Kernel Lab,
// "Decode integration": fixed token/position buffers, then ... the LM-head
// GEMV + argmax + token/position update, all under one graph replay;
// emit_qwen38_generate, "Where the speed comes from", item 2: the sampled
// token and the position advance on the device, so no replay needs a host
// round trip).
//
//  embed_gather : the embedding row of the token the LM-head argmax wrote
//                 (read from device memory), dequantized to f32.
//  token_advance: appends that token to a device token history and
//                 increments the position.
#include "common.hpp"
#include "internal.hpp"

namespace wsg {
namespace {

constexpr int kEmbedThreads = 256;

// out[i] = row `token` of the table, dequantized: a Q8_0 row in the device
// layout (d * q, exact in f32: an 11-bit scale times an 8-bit code) or a
// bf16 row.  A token outside [0, vocab) gives a zero row.
template <bool Q8>
__global__ __launch_bounds__(kEmbedThreads) void embed_gather_kernel(const uint8_t* __restrict__ table, int vocab,
                                                                     int hidden, const int32_t* __restrict__ token,
                                                                     float* __restrict__ out) {
    const int i = (int)(blockIdx.x * kEmbedThreads + threadIdx.x);
    if (i >= hidden) return;
    const int t = *token;
    if (t < 0 || t >= vocab) {
        out[i] = 0.0f;
        return;
    }
    if constexpr (Q8) {
        const int C = (int)chunk_count(hidden);
        const int c = i / kChunkWeights, b = (i % kChunkWeights) / kBlock, j = i % kBlock;
        const bool last = c == C - 1;
        const int nbc = last ? (hidden / kBlock - (C - 1) * kChunkBlocks) : kChunkBlocks;
        const int sb = (int)scale_section_bytes(nbc);
        const uint8_t* base = table + (int64_t)t * packed_row_bytes(hidden) + (int64_t)c * kFullChunkBytes;
        const uint16_t d = *reinterpret_cast<const uint16_t*>(base + 2 * b);
        const int8_t q = (int8_t)base[sb + (j < 16 ? 16 * b + j : 16 * nbc + 16 * b + (j - 16))];
        out[i] = half_bits_to_float(d) * (float)q;
    } else {
        const uint16_t h = reinterpret_cast<const uint16_t*>(table)[(int64_t)t * hidden + i];
        out[i] = __uint_as_float((uint32_t)h << 16);
    }
}

// One thread: history[pos] = token (while pos < capacity), pos += 1.
__global__ void token_advance_kernel(const int32_t* __restrict__ token, int32_t* __restrict__ history,
                                     int capacity, int32_t* __restrict__ pos) {
    const int p = *pos;
    if (p >= 0 && p < capacity) history[p] = *token;
    *pos = p + 1;
}

}  // namespace

int validate_embed_gather(const void* table, int w_type, int64_t vocab, int64_t hidden, const int32_t* token,
                          const float* out) {
    if (w_type != WSG_W_BF16 && w_type != WSG_W_Q8_0) return WSG_ERR_MODE;
    if (vocab < 1 || hidden < 1 || vocab > kMaxDim || hidden > kMaxDim) return WSG_ERR_SHAPE;
    if (w_type == WSG_W_Q8_0 && hidden % kBlock) return WSG_ERR_SHAPE;
    if (!table || !token || !out) return WSG_ERR_NULL;
    if (!aligned(table, 16) || !aligned(token, 4) || !aligned(out, 4)) return WSG_ERR_ALIGN;
    return WSG_OK;
}

int validate_token_advance(const int32_t* token, const int32_t* history, int64_t capacity, const int32_t* pos) {
    if (capacity < 0 || capacity > kMaxDim) return WSG_ERR_SHAPE;
    if (!token || !pos || (capacity > 0 && !history)) return WSG_ERR_NULL;
    if (!aligned(token, 4) || !aligned(pos, 4) || (history && !aligned(history, 4))) return WSG_ERR_ALIGN;
    return WSG_OK;
}

}  // namespace wsg

using namespace wsg;

extern "C" {

int embed_gather(const void* table, int w_type, int64_t vocab, int64_t hidden, const int32_t* token, float* out,
                 hipStream_t stream) {
    const int rc = validate_embed_gather(table, w_type, vocab, hidden, token, out);
    if (rc != WSG_OK) return rc;
    const dim3 grid((unsigned)((hidden + kEmbedThreads - 1) / kEmbedThreads));
    const uint8_t* t = static_cast<const uint8_t*>(table);
    if (w_type == WSG_W_Q8_0) {
        hipLaunchKernelGGL(embed_gather_kernel<true>, grid, dim3(kEmbedThreads), 0, stream, t, (int)vocab,
                           (int)hidden, token, out);
    } else {
        hipLaunchKernelGGL(embed_gather_kernel<false>, grid, dim3(kEmbedThreads), 0, stream, t, (int)vocab,
                           (int)hidden, token, out);
    }
    return launch_status();
}

int token_advance(const int32_t* token, int32_t* history, int64_t capacity, int32_t* pos, hipStream_t stream) {
    const int rc = validate_token_advance(token, history, capacity, pos);
    if (rc != WSG_OK) return rc;
    hipLaunchKernelGGL(token_advance_kernel, dim3(1), dim3(1), 0, stream, token, history, (int)capacity, pos);
    return launch_status();
}

}  // extern "C"
