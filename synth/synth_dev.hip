// Device implementation of the seeded synthetic-input generator, for inputs
// too large to build on the host (multi-GB weight streams).  It implements
// the definition stated in synth.h word for word: the same SplitMix64
// counter stream, the same Irwin-Hall(12) sum of 20-bit fields, and one
// fp32 multiply per element, so its output is byte-identical to synth.c.
// It holds none of the method's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

__host__ __device__ inline uint64_t word(uint64_t key, uint64_t n) { return mix64(key + (n + 1) * kGolden); }

__global__ void normal_fill(uint64_t key, uint64_t first, int64_t count, float scale, float* out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const uint64_t e = first + (uint64_t)i;
        int64_t s = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint64_t w = word(key, 4 * e + (uint64_t)j);
            s += (int64_t)(w & 0xFFFFF);
            s += (int64_t)((w >> 20) & 0xFFFFF);
            s += (int64_t)((w >> 40) & 0xFFFFF);
        }
        const int32_t z = (int32_t)(s - 6 * (int64_t)0xFFFFF);
        out[i] = __fmul_rn((float)z, scale);
    }
}

}  // namespace

extern "C" {

// out[i] = normal(key(seed, tensor), first + i, sigma), i < count, written on
// `stream` (device pointer out, caller-owned).  Returns 0, or 1 on a bad
// argument, or 2 if the launch failed.
int synth_dev_normal_f32(uint64_t seed, uint64_t tensor, int64_t first, int64_t count, float sigma,
                         float* out, hipStream_t stream) {
    if (count < 0 || first < 0 || (count > 0 && out == nullptr)) return 1;
    if (count == 0) return 0;
    const uint64_t key = word(seed, tensor);
    const float scale = sigma * (1.0f / 1048576.0f);
    int64_t blocks = (count + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(normal_fill, dim3((unsigned)blocks), dim3(256), 0, stream, key, (uint64_t)first,
                       count, scale, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
