// Per-workgroup timestamps of the int8 GEMV kernel and of the persistent
// token kernel (per op: see tl_op), for the diagnostic
// build only (build.py --timeline defines WSG_TIMELINE and writes
// libwsgemv_timeline.so; the library proper compiles every macro here to
// nothing).  Each workgroup of each launch records, from the GPU's
// constant 100 MHz clock (s_memrealtime): its entry, the end of its
// activation staging, the first and the last of its waves to finish the
// row loop (and which waves they were), its end, its CU and XCD, and the
// latest wave entry.  A launch
// is told apart by its output pointer: the record of workgroup b of the
// launch writing y goes to slot ((y >> 2) % modulus) * 512 + b of the
// buffer set by wsg_timeline_set (the caller picks a modulus under which
// the outputs it traces do not collide); workgroups from 512 on are not
// recorded.  One vector store per field from thread 0.
#pragma once

#include "common.hpp"

#ifdef WSG_TIMELINE

namespace wsg {

constexpr int kTimelineFields = 10;
constexpr unsigned kTimelineWorkgroups = 512;

// Each source file that records has its own copy (the library is built
// without relocatable device code); wsg_timeline_set sets all of them.
static __device__ uint64_t* g_timeline;
static __device__ uint32_t g_timeline_mod;

static inline int tl_set_here(void* buf, uint32_t modulus) {
    uint64_t* b = static_cast<uint64_t*>(buf);
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_timeline), &b, sizeof(b)) != hipSuccess) return -1;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_timeline_mod), &modulus, sizeof(modulus)) != hipSuccess) return -1;
    return 0;
}
int stream_timeline_set(void* buf, uint32_t modulus);  // stream.hip's copy

__device__ inline uint64_t tl_now() { return __builtin_amdgcn_s_memrealtime(); }

struct TlWaves {
    uint64_t t[16][2];  // per wave: entry, end of the row loop
};
__device__ inline TlWaves& tl_waves() {
    __shared__ TlWaves w;
    return w;
}

__device__ inline void tl_wave(int field, uint64_t t) {
    const unsigned w = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0 && w < 16) tl_waves().t[w][field] = t;
}

__device__ inline void tl_end(uint64_t t_entry, uint64_t t_staged, const void* y) {
    __syncthreads();
    if (threadIdx.x != 0 || g_timeline == nullptr || g_timeline_mod == 0 || blockIdx.x >= kTimelineWorkgroups) return;
    const uint64_t t_end = tl_now();
    const int nw = (int)(blockDim.x / kWave) < 16 ? (int)(blockDim.x / kWave) : 16;
    const TlWaves& w = tl_waves();
    uint64_t first_end = ~0ull, last_end = 0, last_entry = 0;
    uint64_t first_wave = 0, last_wave = 0;
    for (int i = 0; i < nw; ++i) {
        if (w.t[i][1] < first_end) {
            first_end = w.t[i][1];
            first_wave = (uint64_t)i;
        }
        if (w.t[i][1] > last_end) {
            last_end = w.t[i][1];
            last_wave = (uint64_t)i;
        }
        last_entry = w.t[i][0] > last_entry ? w.t[i][0] : last_entry;
    }
    const uint64_t key = ((uint64_t)y >> 2) % g_timeline_mod;
    uint64_t* r = g_timeline + (key * kTimelineWorkgroups + blockIdx.x) * kTimelineFields;
    r[0] = (uint64_t)y;
    r[1] = blockIdx.x | ((uint64_t)gridDim.x << 32);
    r[2] = t_entry;
    r[3] = t_staged;
    r[4] = first_end;
    r[5] = last_end;
    r[6] = t_end;
    r[7] = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID: CU, SE
    // XCC_ID, and the waves that ended the row loop first and last
    r[8] = __builtin_amdgcn_s_getreg((31 << 11) | 20) | (first_wave << 32) | (last_wave << 40);
    r[9] = last_entry;
}

// The persistent token kernel records one slot per op and workgroup: slot
// op * 512 + b (the caller sizes the buffer for every op; the modulus is not
// used).  Fields: 0 the op index, 1 blk | grid << 32, 2 when the op's first
// weight requests were issued (the previous op's results stored, or the
// kernel's entry), 3 the op's input staged, 4 the row loop ended (every
// wave: after the barrier), 5 the op's results stored (thread 0's share),
// 7 HW_ID, 8 XCC_ID.
__device__ inline void tl_op(int op, int field, uint64_t t) {
    if (threadIdx.x != 0 || g_timeline == nullptr || blockIdx.x >= kTimelineWorkgroups) return;
    uint64_t* r = g_timeline + ((uint64_t)op * kTimelineWorkgroups + blockIdx.x) * kTimelineFields;
    if (field == 2) {
        r[0] = (uint64_t)op;
        r[1] = blockIdx.x | ((uint64_t)gridDim.x << 32);
        r[7] = __builtin_amdgcn_s_getreg((31 << 11) | 4);
        r[8] = __builtin_amdgcn_s_getreg((31 << 11) | 20);
    }
    r[field] = t;
}

}  // namespace wsg

#define WSG_TL_OP(op, field) wsg::tl_op((op), (field), wsg::tl_now())
#define WSG_TL_BEGIN()                          \
    const uint64_t tl_t_entry = wsg::tl_now(); \
    wsg::tl_wave(0, tl_t_entry)
#define WSG_TL_STAGED() const uint64_t tl_t_staged = wsg::tl_now()
#define WSG_TL_LOOP_END() wsg::tl_wave(1, wsg::tl_now())
#define WSG_TL_END(y) wsg::tl_end(tl_t_entry, tl_t_staged, (y))

#else

#define WSG_TL_OP(op, field) (void)0
#define WSG_TL_BEGIN() (void)0
#define WSG_TL_STAGED() (void)0
#define WSG_TL_LOOP_END() (void)0
#define WSG_TL_END(y) (void)0

#endif
