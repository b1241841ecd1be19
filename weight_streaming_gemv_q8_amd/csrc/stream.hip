// Persistent whole-token kernel: one launch runs a token's whole chain of
// Q8_0 GEMVs (emit_qwen38_generate, "Where the speed comes from", items 1-2:
// the GEMV weight stream is ~90% of a decode step and must not stall between
// launches).  A launch per GEMV pays a ramp (first requests in flight) and a
// tail (last workgroups finishing) every time; here every workgroup stays
// resident, requests the next matrix's first weights as soon as it has
// finished its rows of the current one (weights do not depend on the
// activation), and only then waits at a grid-wide barrier for the activation
// that the next GEMV reads.
//
// Barrier: each workgroup posts an arrival epoch in its own cache line,
// workgroup 0 collects them and posts a release epoch (see below).  A wait
// that exceeds its spin limit sets an error flag and gives up, so every wave
// always exits.  The grid never exceeds the number of co-resident
// workgroups.
#include "common.hpp"
#include "gemv_device.hpp"
#include "internal.hpp"
#include "stream.hpp"

namespace wsg {
namespace {

constexpr int kStreamWaves = 8;

// Descriptor pointers are read from memory, so the compiler cannot tell they
// point to global memory and would use flat instructions, which also count
// against the LDS wait counter: the barrier would then wait for the weight
// prefetch.  The weight pointer is therefore carried as a global pointer.
constexpr int kStreamUnroll = 2;

// ------------------------------------------------------------ barrier
// Device-scope coherence without cache maintenance: outputs that another
// workgroup reads later are written with device-scope stores (visible at
// device level once complete) and read with device-scope loads, so no L2
// write-back or invalidation is needed at a barrier.
//
// Barrier state (uint32 words, each group on its own 128-byte line):
//   st[0]              launch counter (read at start, bumped by workgroup 0 at the end)
//   st[32]             release epoch, written by workgroup 0
//   st[64]             error flag
//   st[96 + 32 * w]    arrival epoch of workgroup w
// Barrier b of a launch uses epoch = launch * 4096 + b + 1.
constexpr int kBarRelease = 32, kBarError = 64, kBarArrive = 96, kBarStride = 32;

__device__ inline uint32_t ld_dev(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until this wave's outstanding vector-memory operations (its
// device-scope output stores) have completed.
__device__ inline void drain_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Arrive: every wave has drained its stores; thread 0 posts the epoch.
__device__ inline void barrier_arrive(uint32_t* st, uint32_t epoch) {
    drain_vmem();
    __syncthreads();
    if (threadIdx.x == 0) st_dev(st + kBarArrive + kBarStride * blockIdx.x, epoch);
}

// Wait: workgroup 0 collects every arrival (one thread per workgroup) and
// posts the release; everyone waits for it.  Each poll is bounded.
__device__ inline void barrier_wait(uint32_t* st, uint32_t epoch, int spin_limit) {
    if (blockIdx.x == 0) {
        int spins = 0;  // one budget per thread for all of its flags
        for (int w = threadIdx.x; w < (int)gridDim.x; w += blockDim.x) {
            const uint32_t* f = st + kBarArrive + kBarStride * w;
            while (ld_dev(f) != epoch) {
                __builtin_amdgcn_s_sleep(1);
                if (++spins >= spin_limit) {
                    st_dev(st + kBarError, 1u);
                    break;
                }
            }
            if (spins >= spin_limit) break;
        }
        __syncthreads();
        if (threadIdx.x == 0) st_dev(st + kBarRelease, epoch);
    }
    if (threadIdx.x == 0) {
        int spins = 0;
        while (ld_dev(st + kBarRelease) != epoch) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins >= spin_limit) {
                st_dev(st + kBarError, 1u);
                break;
            }
        }
    }
    __syncthreads();
}

// Device-scope loads of an f32 activation written by other workgroups in
// this launch (8 bytes per load).
__device__ inline float4v ld_dev_f4(const float* p) {
    const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float4v v;
    v.x = __uint_as_float((uint32_t)a);
    v.y = __uint_as_float((uint32_t)(a >> 32));
    v.z = __uint_as_float((uint32_t)b);
    v.w = __uint_as_float((uint32_t)(b >> 32));
    return v;
}

// Stage the activation with device-scope loads (requantized, or f32).
__device__ inline void stage_requant_dev(const float* x, int k, int4v* lds_q, float* lds_dx) {
    const int NB = k / kBlock;
    for (int b = threadIdx.x; b < NB; b += blockDim.x) {
        float4v t[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) t[g] = ld_dev_f4(x + (int64_t)b * kBlock + 4 * g);
        requant_block_to_lds(t, b, lds_q, lds_dx);
    }
}

__device__ inline void stage_f32_dev(const float* x, int k, float4v* lds_x) {
    for (int u = threadIdx.x; u < k / 4; u += blockDim.x) lds_x[StageF32<1>::slot(u)] = ld_dev_f4(x + 4 * u);
}

// Split-K epilogue with a run-time split factor.
__device__ inline void finish_row_rt(float acc, int row, int n, int S, float* lds_part, float* y) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int part = wave % S;
    float total = acc;
    if (S > 1) {
        if (lane == 0) lds_part[wave] = acc;
        __syncthreads();
        if (part == 0) {
            total = lds_part[wave];
            for (int p = 1; p < S; ++p) total += lds_part[wave + p];
        }
        __syncthreads();
    }
    if (part == 0 && row < n && lane == 0)
        __hip_atomic_store(y + row, total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int WAVES, int U, bool F32>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(4)))
stream_kernel(const StreamOp* __restrict__ ops, int n_ops, uint32_t* __restrict__ st, int spin_limit) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ uint32_t launch_id;
    if (threadIdx.x == 0) launch_id = ld_dev(st);
    __syncthreads();
    uint32_t epoch = launch_id * 4096u;
    for (int j = 0; j < n_ops; ++j) {
        const StreamOp op = ops[j];
        const gptr<uint8_t> opw = (gptr<uint8_t>)op.w;
        const int n = op.n, k = op.k, S = op.split;
        const int C = (int)chunk_count(k);
        const int NB = k / kBlock;
        const int nl = NB - (C - 1) * kChunkBlocks;
        const int sbl = (int)scale_section_bytes(nl);
        const int64_t row_bytes = packed_row_bytes(k);
        const size_t act_bytes = F32 ? lds_f32act_bytes(C) : lds_q8act_bytes(C);
        float* lds_part = reinterpret_cast<float*>(smem + act_bytes);
        const float4v* lds_x = reinterpret_cast<const float4v*>(smem);
        const int4v* lds_q = reinterpret_cast<const int4v*>(smem);
        const float* lds_dx = reinterpret_cast<const float*>(smem + (size_t)C * 2 * kWave * 16);

        const Sched sc(C, S, U, WAVES, n, (n + WAVES / S - 1) / (WAVES / S));
        auto load = [&](Q8Regs<U>& r, int row, int m) { q8_load<U>(r, opw, row_bytes, sc, nl, sbl, row, m); };

        // arrive (outputs drained), request the next matrix's first weights,
        // then wait for everyone else's outputs
        Q8Regs<U> cur;
        if (op.barrier) {
            ++epoch;
            barrier_arrive(st, epoch);
            if (sc.tiles_wg > 0 && sc.ipt > 0 && sc.row(0) < n) load(cur, sc.row(0), 0);
            barrier_wait(st, epoch, spin_limit);
        } else {
            if (sc.tiles_wg > 0 && sc.ipt > 0 && sc.row(0) < n) load(cur, sc.row(0), 0);
            __syncthreads();  // the previous op's LDS contents are dead
        }

        if constexpr (F32) {
            stage_f32_dev(op.x, k, reinterpret_cast<float4v*>(smem));
        } else {
            stage_requant_dev(op.x, k, reinterpret_cast<int4v*>(smem),
                              reinterpret_cast<float*>(smem + (size_t)C * 2 * kWave * 16));
        }
        __syncthreads();

        auto compute = [&](const Q8Regs<U>& r, int row, int m, float& acc) {
            if constexpr (F32) {
                q8_f32_item<U>(r, sc, m, NB, lds_x, acc);
            } else {
                q8_i8_item<U, false>(r, sc, m, NB, lds_q, lds_dx, row, nullptr, acc);
            }
        };
        row_loop(sc, cur, load, compute,
                 [&](float acc, int row, bool) { finish_row_rt(acc, row, n, S, lds_part, op.y); });
    }
    // the next launch uses fresh epochs; every workgroup read the counter
    // before its first arrival, and workgroup 0 gets here only after the
    // last barrier
    if (blockIdx.x == 0 && threadIdx.x == 0) st_dev(st, launch_id + 1u);
}

}  // namespace

template <bool F32>
const void* stream_kernel_ptr() {
    return reinterpret_cast<const void*>(stream_kernel<kStreamWaves, F32 ? 1 : kStreamUnroll, F32>);
}

int stream_config(int max_k, bool f32, int* waves, int* grid, size_t* lds) {
    const void* kern = f32 ? stream_kernel_ptr<true>() : stream_kernel_ptr<false>();
    const int C = (int)chunk_count(max_k);
    const size_t act = f32 ? lds_f32act_bytes(C) : lds_q8act_bytes(C);
    const size_t bytes = act + kStreamWaves * sizeof(float) + 16;
    if (bytes > 65536) (void)hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kStreamWaves * kWave, bytes) != hipSuccess ||
        per_cu < 1)
        return WSG_ERR_HIP;
    *waves = kStreamWaves;
    *grid = device_info().cus * per_cu;
    *lds = bytes;
    return WSG_OK;
}

int stream_launch(const StreamOp* ops_dev, int n_ops, bool f32, uint32_t* bar_dev, int grid, size_t lds,
                  int spin_limit, hipStream_t stream) {
    if (f32) {
        hipLaunchKernelGGL((stream_kernel<kStreamWaves, 1, true>), dim3(grid), dim3(kStreamWaves * kWave), lds,
                           stream, ops_dev, n_ops, bar_dev, spin_limit);
    } else {
        hipLaunchKernelGGL((stream_kernel<kStreamWaves, kStreamUnroll, false>), dim3(grid),
                           dim3(kStreamWaves * kWave), lds, stream, ops_dev, n_ops, bar_dev, spin_limit);
    }
    return launch_status();
}

int stream_split(bool f32, int64_t n, int64_t k) {
    const int s = gemv_split(f32, n, k);
    return s > kStreamWaves ? kStreamWaves : s;
}

}  // namespace wsg
