// Measurement kernels: an HBM read-ceiling probe that streams a buffer with
// the GEMV's load width and cache policy, and a copy kernel of exactly known
// traffic used to calibrate the hardware byte counters.
#include "common.hpp"
#include "internal.hpp"

namespace wsg {
namespace {

// Each wave streams one contiguous span of the buffer (whole 1 KB wave
// loads, U in flight), the pattern that measured fastest on this part
// (~7 TB/s over 8 GiB with four 4-wave workgroups per CU, against ~6.3-6.5
// for a grid-stride loop over the whole buffer).
template <int U>
__global__ void __launch_bounds__(256) read_probe_kernel(const int4v* __restrict__ buf, int64_t n16,
                                                         float* __restrict__ sink) {
    const int lane = (int)threadIdx.x % kWave;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
    const int64_t wid = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t per = ((n16 + waves - 1) / waves + kWave - 1) / kWave * kWave;  // 16-byte units per wave
    const int64_t b = wid * per;
    const int64_t e = b + per < n16 ? b + per : n16;
    int acc = 0;
    int64_t i = b;
    for (; i + (int64_t)kWave * U <= e; i += (int64_t)kWave * U) {
        int4v v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = load16<true>(buf + i + kWave * u + lane);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < e; i += kWave) {
        if (i + lane < e) {
            const int4v v = load16<true>(buf + i + lane);
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    // fold the lanes so that no load can be dropped; one store per workgroup
    acc = (int)wave_sum((float)(acc & 1));
    __shared__ int lds[4];
    if (threadIdx.x % kWave == 0) lds[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = (float)(lds[0] + lds[1] + lds[2] + lds[3]);
}

__global__ void __launch_bounds__(256) copy_probe_kernel(const int4v* __restrict__ src, int4v* __restrict__ dst,
                                                         int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace
}  // namespace wsg

using namespace wsg;

extern "C" {

int wsg_read_probe(const void* buf, int64_t bytes, float* sink, int blocks, hipStream_t stream) {
    if (bytes <= 0 || bytes % 16) return WSG_ERR_SHAPE;
    if (!buf || !sink) return WSG_ERR_NULL;
    if (!aligned(buf, 16) || !aligned(sink, 4)) return WSG_ERR_ALIGN;
    if (blocks <= 0) blocks = device_info().cus * 4;
    hipLaunchKernelGGL(read_probe_kernel<8>, dim3(blocks), dim3(256), 0, stream, static_cast<const int4v*>(buf),
                       bytes / 16, sink);
    return launch_status();
}

int wsg_copy_probe(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    if (bytes <= 0 || bytes % 16) return WSG_ERR_SHAPE;
    if (!src || !dst) return WSG_ERR_NULL;
    if (!aligned(src, 16) || !aligned(dst, 16)) return WSG_ERR_ALIGN;
    const int blocks = device_info().cus * 8;
    hipLaunchKernelGGL(copy_probe_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const int4v*>(src),
                       static_cast<int4v*>(dst), bytes / 16);
    return launch_status();
}

}  // extern "C"
