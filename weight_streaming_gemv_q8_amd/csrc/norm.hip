// The step either side of every GEMV in a decode layer: the residual add,
// the next RMSNorm and the activation re-quantization in one kernel
// (emit_qwen38_generate, "Where the speed comes from", item 3; GPU Kernel
// Lab, "Decode integration": RMSNorm with an FP32 reduction and residual
// fusion).
//
//   h'  = h + r            one fp32 add per element (r absent: h' = h)
//   y_i = h'_i * s * g_i   s = 1 / sqrt(mean_j h'_j^2 + eps), fp32
//   y_q8 = Q8_0(y)         the rule of quantize_act_q8_0, same bytes
//
// At decode the vector is a few KB to a few tens of KB, so the kernel is
// latency-bound, not bandwidth-bound: ONE workgroup does it with a single
// round trip to memory.  Every thread owns "units" of eight consecutive
// values (thread t: units t, t + T, t + 2T, ... for T threads), reads h, r
// and g for all of them up front, keeps h' in registers across the
// reduction and writes each output once.  Four consecutive lanes hold the
// four units of one 32-value block, so the Q8_0 block maximum is a quad
// reduction (q8_quad_codes) and each lane stores its eight codes as one
// 8-byte store.  The mean of squares is reduced in a fixed order: each
// thread over its units, a butterfly over the wave, then the wave partials
// in wave order, so the result does not depend on timing.
#include "common.hpp"
#include "gemv_device.hpp"
#include "internal.hpp"

namespace wsg {
namespace {

constexpr int kNormThreads = 1024;
constexpr int kNormWaves = kNormThreads / kWave;
constexpr int kNormMaxUnits = WSG_MAX_K_Q8ACT / (8 * kNormThreads);  // units per thread: 7
static_assert(kNormMaxUnits * 8 * kNormThreads == WSG_MAX_K_Q8ACT, "k limit is a whole number of units");

// h and r are not __restrict__: h_out may be either of them (an in-place
// residual update); each thread reads its own elements before writing them
// and reads no other thread's.
template <int NU>
__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_kernel(
    const float* h, const float* r, const float* __restrict__ g, int k, float eps, float* h_out,
    float* __restrict__ y, int8_t* __restrict__ q, uint16_t* __restrict__ d, int nt) {
    // g is loaded with h and r while it fits in registers beside h'.
    constexpr bool kEarlyG = NU <= 4;
    __shared__ float wave_part[kNormWaves];
    const int units = k >> 3;
    // nt = the block size, passed as an argument: reading blockDim.x is a
    // vector load on this target, and the first unit's address would wait for it
    const int t = threadIdx.x;

    float a[NU][8];
    float gv[kEarlyG ? NU : 1][8];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        const int u = t + i * nt;
        if (u < units) {
            const float4v* h4 = reinterpret_cast<const float4v*>(h) + 2 * u;
            float4v x0 = h4[0], x1 = h4[1];
            if (r) {
                const float4v* r4 = reinterpret_cast<const float4v*>(r) + 2 * u;
                x0 += r4[0];
                x1 += r4[1];
            }
            if constexpr (kEarlyG) {
                if (g) {
                    const float4v* g4 = reinterpret_cast<const float4v*>(g) + 2 * u;
                    const float4v g0 = g4[0], g1 = g4[1];
                    gv[i][0] = g0.x, gv[i][1] = g0.y, gv[i][2] = g0.z, gv[i][3] = g0.w;
                    gv[i][4] = g1.x, gv[i][5] = g1.y, gv[i][6] = g1.z, gv[i][7] = g1.w;
                }
            }
            if (h_out) {
                float4v* o4 = reinterpret_cast<float4v*>(h_out) + 2 * u;
                o4[0] = x0;
                o4[1] = x1;
            }
            a[i][0] = x0.x, a[i][1] = x0.y, a[i][2] = x0.z, a[i][3] = x0.w;
            a[i][4] = x1.x, a[i][5] = x1.y, a[i][6] = x1.z, a[i][7] = x1.w;
#pragma unroll
            for (int j = 0; j < 8; ++j) ss = __builtin_fmaf(a[i][j], a[i][j], ss);
        }
    }

    ss = wave_sum(ss);
    const int wave = t / kWave;
    if (t % kWave == 0) wave_part[wave] = ss;
    __syncthreads();
    float total = 0.0f;
    for (int w = 0; w < nt / kWave; ++w) total += wave_part[w];
    const float s = 1.0f / __builtin_sqrtf(total / (float)k + eps);

#pragma unroll
    for (int i = 0; i < NU; ++i) {
        const int u = t + i * nt;
        if (u < units) {
            float v[8];
            if (g) {
                float gu[8];
                if constexpr (kEarlyG) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) gu[j] = gv[i][j];
                } else {
                    const float4v* g4 = reinterpret_cast<const float4v*>(g) + 2 * u;
                    const float4v g0 = g4[0], g1 = g4[1];
                    gu[0] = g0.x, gu[1] = g0.y, gu[2] = g0.z, gu[3] = g0.w;
                    gu[4] = g1.x, gu[5] = g1.y, gu[6] = g1.z, gu[7] = g1.w;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = (a[i][j] * s) * gu[j];
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = a[i][j] * s;
            }
            if (y) {
                float4v* y4 = reinterpret_cast<float4v*>(y) + 2 * u;
                y4[0] = float4v{v[0], v[1], v[2], v[3]};
                y4[1] = float4v{v[4], v[5], v[6], v[7]};
            }
            if (q) {
                uint32_t lo, hi;
                const uint16_t d16 = q8_quad_codes(v, lo, hi);
                typedef uint32_t uint2v __attribute__((ext_vector_type(2)));
                *reinterpret_cast<uint2v*>(q + 8 * (int64_t)u) = uint2v{lo, hi};
                if ((u & 3) == 0) d[u >> 2] = d16;
            }
        }
    }
}

template <int NU>
void launch_norm(int threads, hipStream_t s, const float* h, const float* r, const float* g, int k, float eps,
                 float* h_out, float* y, int8_t* q, uint16_t* d) {
    hipLaunchKernelGGL(residual_rmsnorm_kernel<NU>, dim3(1), dim3(threads), 0, s, h, r, g, k, eps, h_out, y, q, d,
                       threads);
}

// Threads and units per thread the kernel uses for a vector of k values
// (norm_threads: a GEMV that computes this step in its prologue plays the
// same threads).
void norm_shape(int64_t k, int* threads, int* units_per_thread) {
    const int nt = norm_threads((int)k);
    *threads = nt;
    *units_per_thread = (int)((k / 8 + nt - 1) / nt);
}

}  // namespace

// Argument checks of residual_rmsnorm_q8_0 (also run by the plan before
// capture).
int validate_residual_rmsnorm(const float* h, const float* r, const float* g, int64_t k, float eps,
                              const void* h_out, const void* y, const void* y_q8) {
    if (k < 0 || k > WSG_MAX_K_Q8ACT || k % kBlock) return WSG_ERR_SHAPE;
    if (!(eps > 0.0f) || !(eps < __builtin_inff())) return WSG_ERR_MODE;
    if (k == 0 || (!h_out && !y && !y_q8)) return WSG_OK;
    if (!h) return WSG_ERR_NULL;
    if (!aligned(h, 16) || (r && !aligned(r, 16)) || (g && !aligned(g, 16)) || (h_out && !aligned(h_out, 16)) ||
        (y && !aligned(y, 16)) || (y_q8 && !aligned(y_q8, 16)))
        return WSG_ERR_ALIGN;
    return WSG_OK;
}

}  // namespace wsg

using namespace wsg;

extern "C" {

int residual_rmsnorm_q8_0(const float* h, const float* r, const float* g, int64_t k, float eps, float* h_out,
                          float* y, void* y_q8, hipStream_t stream) {
    const int rc = validate_residual_rmsnorm(h, r, g, k, eps, h_out, y, y_q8);
    if (rc != WSG_OK || k == 0 || (!h_out && !y && !y_q8)) return rc;
    int threads, nu;
    norm_shape(k, &threads, &nu);
    int8_t* q = static_cast<int8_t*>(y_q8);
    uint16_t* d = q ? reinterpret_cast<uint16_t*>(q + k) : nullptr;
    const int kk = (int)k;
    switch (nu) {
        case 1: launch_norm<1>(threads, stream, h, r, g, kk, eps, h_out, y, q, d); break;
        case 2: launch_norm<2>(threads, stream, h, r, g, kk, eps, h_out, y, q, d); break;
        case 3: launch_norm<3>(threads, stream, h, r, g, kk, eps, h_out, y, q, d); break;
        case 4: launch_norm<4>(threads, stream, h, r, g, kk, eps, h_out, y, q, d); break;
        case 5: launch_norm<5>(threads, stream, h, r, g, kk, eps, h_out, y, q, d); break;
        case 6: launch_norm<6>(threads, stream, h, r, g, kk, eps, h_out, y, q, d); break;
        case 7: launch_norm<7>(threads, stream, h, r, g, kk, eps, h_out, y, q, d); break;
        default: return WSG_ERR_SHAPE;
    }
    return launch_status();
}

}  // extern "C"
