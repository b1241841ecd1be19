// Does a line touched by one kernel stay in its XCD's L2 for the next kernel
// on the same stream?  A standalone diagnostic program (not part of the
// library): each workgroup b of 64 threads owns region b of 16 KB (128 lines
// of 128 B) of a 4 MB buffer.  The probe kernel times, with the GPU's 100 MHz
// constant clock, its workgroup's first pass over one dword per line and a
// second pass over the same lines (an L2 hit), after: a 1 GB sweep (cold);
// a touch of the same lines by the previous kernel; that touch followed by a
// 64 MB sweep kernel (evicts L2, not the memory-side cache).  Workgroup b
// runs on the same XCD in every kernel (dispatch deals workgroups to XCDs
// round robin), so the touch and the probe meet in one L2.
//
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       -o l2keep weight_streaming_gemv_q8_amd/diag/l2keep.hip && ./l2keep
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
#include <algorithm>
#define CHECK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)
constexpr int kWG = 256, kRegion = 16384;

__global__ void touch(const unsigned* __restrict__ buf, unsigned* sink) {
    const unsigned* r = buf + (size_t)blockIdx.x * (kRegion / 4);
    unsigned s = 0;
    for (int i = threadIdx.x; i < kRegion / 128; i += 64) s += r[i * 32];  // one dword per 128-B line
    if (s == 0xFFFFFFFFu) sink[blockIdx.x] = s;
}
// times[b*2+0] = first pass latency (ticks), [b*2+1] = second pass (same lines, now surely in L2)
__global__ void probe(const unsigned* __restrict__ buf, unsigned* sink, unsigned long long* times) {
    const unsigned* r = buf + (size_t)blockIdx.x * (kRegion / 4);
    unsigned s = 0;
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    for (int i = threadIdx.x; i < kRegion / 128; i += 64) s += __builtin_nontemporal_load(r + i * 32);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
    for (int i = threadIdx.x; i < kRegion / 128; i += 64) s += __builtin_nontemporal_load(r + i * 32 + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const unsigned long long t2 = __builtin_amdgcn_s_memrealtime();
    if (s == 0xFFFFFFFFu) sink[blockIdx.x] = s;
    if (threadIdx.x == 0) { times[2 * blockIdx.x] = t1 - t0; times[2 * blockIdx.x + 1] = t2 - t1; }
}
// streams a large buffer (evicts L2; 64 MB stays in the memory-side cache)
__global__ void sweep(const uint4* __restrict__ big, size_t n16, unsigned* sink) {
    uint4 a = make_uint4(0, 0, 0, 0);
    for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) {
        uint4 v = big[i]; a.x ^= v.x; a.y ^= v.y; a.z ^= v.z; a.w ^= v.w;
    }
    if ((a.x & a.y & a.z & a.w) == 0xFFFFFFFFu) sink[0] = a.x;
}

int main() {
    const size_t region_bytes = (size_t)kWG * kRegion;           // 4 MB probed
    const size_t big_bytes = (size_t)1 << 30, mid_bytes = (size_t)64 << 20;
    unsigned *buf, *sink; uint4 *big; unsigned long long* times;
    CHECK(hipMalloc(&buf, region_bytes)); CHECK(hipMalloc(&sink, kWG * 4)); CHECK(hipMalloc(&big, big_bytes));
    CHECK(hipMalloc(&times, kWG * 16));
    CHECK(hipMemset(buf, 1, region_bytes)); CHECK(hipMemset(big, 2, big_bytes));
    CHECK(hipDeviceSynchronize());
    std::vector<unsigned long long> h(kWG * 2);
    auto run = [&](const char* name, int mode) -> int {
        double first = 0, second = 0;
        std::vector<double> f, sc;
        for (int rep = 0; rep < 5; ++rep) {
            sweep<<<1024, 256>>>(big, big_bytes / 16, sink);                 // evict L2 and the MALL
            if (mode == 1) touch<<<kWG, 64>>>(buf, sink);                     // touch, probe next
            if (mode == 2) { touch<<<kWG, 64>>>(buf, sink); sweep<<<1024, 256>>>(big, mid_bytes / 16, sink); }
            probe<<<kWG, 64>>>(buf, sink, times);
            if (hipDeviceSynchronize() != hipSuccess) return 1;
            if (hipMemcpy(h.data(), times, kWG * 16, hipMemcpyDeviceToHost) != hipSuccess) return 1;
            std::vector<double> a, b;
            for (int i = 0; i < kWG; ++i) { a.push_back(h[2 * i] * 10.0); b.push_back(h[2 * i + 1] * 10.0); }
            std::sort(a.begin(), a.end()); std::sort(b.begin(), b.end());
            f.push_back(a[kWG / 2]); sc.push_back(b[kWG / 2]);
        }
        std::sort(f.begin(), f.end()); std::sort(sc.begin(), sc.end());
        printf("%-40s first pass median %7.0f ns, second pass (L2 hit) %7.0f ns\n", name, f[2], sc[2]);
        return 0;
    };
    if (run("cold (after a 1 GB sweep)", 0)) return 1;
    if (run("touched by the previous kernel", 1)) return 1;
    if (run("touched, then a 64 MB sweep kernel", 2)) return 1;
    CHECK(hipFree(buf)); CHECK(hipFree(sink)); CHECK(hipFree(big)); CHECK(hipFree(times));
    return 0;
}
