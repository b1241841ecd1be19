// Persistent whole-token kernel: one launch runs a token's whole chain of
// Q8_0 GEMVs (emit_qwen38_generate, "Where the speed comes from", items 1-2:
// the GEMV weight stream is ~90% of a decode step and must not stall between
// launches).  A launch per GEMV pays a ramp (first requests in flight) and a
// tail (last workgroups finishing) every time; here one 16-wave workgroup
// per CU stays resident for the whole token.  When a workgroup has finished
// its rows of one GEMV and stored them, it requests the first three items of
// weights of the next GEMV (weights do not depend on the activation) and
// only then waits for that GEMV's activation, so the weight stream keeps HBM
// busy across the wait and the staging of the activation.  (Requesting them
// earlier -- before the stores, or while the last rows are still computed --
// measured slower: the stores and the stragglers' loads then queue behind
// them, and the stores of the last workgroup are what every other one waits
// for.)
//
// Dataflow instead of grid barriers: every GEMV output row is also written
// into a copy that the plan owns, double-buffered by launch parity: the
// value goes into this launch's buffer and a signalling-NaN sentinel into
// the other one, which the next launch will fill.  Arithmetic never returns
// a signalling NaN, so a GEMV whose input is an earlier GEMV's output stages
// it from the copy and re-reads any element that still holds the sentinel:
// an element is read only once its row is written, nothing waits for
// stores to be acknowledged and no counter is shared.  (The buffer a launch
// reads was reset by the previous launch, which had finished reading the
// values of the launch before.)  The parity comes from a 64-bit launch
// counter that every workgroup increments once at start (old value / grid:
// all workgroups of a launch draw the same number).  Every wait is bounded:
// on the spin limit a workgroup sets an error flag, and every wait polls
// that flag now and then, so every wave always exits; the plan reports the
// flag.  The grid never exceeds the number of co-resident workgroups (one
// per CU), so a producer is never waiting for a CU that a waiting consumer
// holds.
#include "common.hpp"
#include "gemv_device.hpp"
#include "internal.hpp"
#include "stream.hpp"
#include "timeline.hpp"

namespace wsg {
namespace {

// One 16-wave workgroup per CU (four waves per SIMD, at most 128 VGPRs
// each), each wave with a ring of three items of one chunk each: two in
// flight while the third is consumed.  (Eight waves per CU stream ~25%
// slower: too few waves to hide the latency of the compute's own LDS reads.
// Deeper rings, or two chunks per item, measured slower: the activation
// staging at each op start waits for every weight load issued before it,
// since loads complete in order.)
constexpr int kStreamWaves = 16;
constexpr int kStreamUnroll = 1;
constexpr int kStreamSets = 3;
constexpr int kStreamThreads = kStreamWaves * kWave;
// Plan state, in uint32 words (each on its own 128-byte line): a 64-bit
// launch counter, the error flag.
constexpr int kStCounter = 0, kStError = 32, kStDetail = 33, kStWords = 64;
// Sites of a wait that gave up (word kStDetail).
constexpr int kSiteStaging = 1;  // an input or dependency not written in time
// Most row tiles one workgroup takes in one op: the tiles' results wait in
// LDS until the op's end.
constexpr int kMaxTiles = 64;
// How often (in polls) a waiting thread also looks at the error flag.
constexpr int kErrorPollMask = 255;

__device__ inline uint32_t ld_dev(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Activation pointers are read from the descriptor table; they are carried
// as global-address-space pointers so that their loads and stores are
// global (not flat) instructions, which do not count against the LDS wait
// counter.
typedef const __attribute__((address_space(1))) float* gcfloat;
typedef __attribute__((address_space(1))) float* gfloat;
typedef const __attribute__((address_space(1))) uint64_t* gcu64;
typedef const __attribute__((address_space(1))) uint32_t* gcu32;

__device__ inline uint64_t ld_dev64(gcu64 p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// "Not written yet": a signalling NaN, which no arithmetic result can be.
constexpr uint32_t kSentinel = kStreamSentinel;
__device__ inline bool ready(float v) { return __float_as_uint(v) != kSentinel; }
__device__ inline bool ready4(float4v v) { return ready(v.x) && ready(v.y) && ready(v.z) && ready(v.w); }

// One round of a bounded wait: counts a poll, gives up on the spin limit or
// when another wait has given up (the error flag, looked at now and then).
// Returns false when the caller must stop waiting.  The first wait of a
// launch to reach its limit also records where it was: the site code, the
// workgroup, the wave and three site-specific values (kStDetail words).
__device__ inline bool poll_again(uint32_t* st, int spin_limit, int& spins, int site = kSiteStaging, int a = 0,
                                  int b = 0, int c = 0) {
    if (++spins >= spin_limit) {
        uint32_t none = 0u;
        if (__hip_atomic_compare_exchange_strong(st + kStDetail, &none, (uint32_t)site, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            st_dev(st + kStDetail + 1, blockIdx.x);
            st_dev(st + kStDetail + 2, threadIdx.x / kWave);
            st_dev(st + kStDetail + 3, (uint32_t)a);
            st_dev(st + kStDetail + 4, (uint32_t)b);
            st_dev(st + kStDetail + 5, (uint32_t)c);
        }
        st_dev(st + kStError, 1u);
        return false;
    }
    if ((spins & kErrorPollMask) == 0 && ld_dev(st + kStError) != 0u) {
        spins = spin_limit;  // results are invalid already: stop waiting
        return false;
    }
    __builtin_amdgcn_s_sleep(1);
    return true;
}

// Device-scope loads of an f32 input written before the launch (8 bytes per
// load).
__device__ inline float4v ld_dev_f4(gcfloat p) {
    const gcu64 q = reinterpret_cast<gcu64>(p);
    const uint64_t a = ld_dev64(q);
    const uint64_t b = ld_dev64(q + 1);
    float4v v;
    v.x = __uint_as_float((uint32_t)a);
    v.y = __uint_as_float((uint32_t)(a >> 32));
    v.z = __uint_as_float((uint32_t)b);
    v.w = __uint_as_float((uint32_t)(b >> 32));
    return v;
}

// Staging of op inputs.  A unit is eight values (requantized path: four
// lanes per 32-value block) or four values (f32 path).  Each thread first
// requests all of its units (up to NR rounds of the workgroup) and then
// converts them, so the staging costs one round trip when the input is
// ready.  An input produced in this launch is read from the producer's copy;
// each round re-requests every group of four values that still holds a
// sentinel, so a round costs one round trip however many are missing.
// T threads share the work (thread tid of them).
template <int NR, int G, int T>
__device__ inline void issue_units(gcfloat src, int base, int units, float4v (&v)[NR][G], int tid) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int u = base + tid + i * T;
        if (u < units) {
#pragma unroll
            for (int q = 0; q < G; ++q) v[i][q] = ld_dev_f4(src + (int64_t)4 * (G * u + q));
        }
    }
}

// Requests again every group of four values that still holds a sentinel
// (unrolled by recursion, so v is indexed by constants and stays in
// registers).
template <int I, int NR, int G, int T>
struct RetryUnits {
    __device__ static void run(gcfloat src, int base, int units, float4v (&v)[NR][G], int tid) {
        if constexpr (I < NR) {
            const int u = base + tid + I * T;
            if (u < units && !ready4(v[I][0])) v[I][0] = ld_dev_f4(src + (int64_t)4 * (G * u));
            if constexpr (G > 1) {
                if (u < units && !ready4(v[I][1])) v[I][1] = ld_dev_f4(src + (int64_t)4 * (G * u + 1));
            }
            RetryUnits<I + 1, NR, G, T>::run(src, base, units, v, tid);
        }
    }
};

template <int NR, int G, int T>
__device__ inline void await_units(gcfloat src, int base, int units, float4v (&v)[NR][G], uint32_t* st,
                                   int spin_limit, int& spins, int tid) {
    for (;;) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = base + tid + i * T;
#pragma unroll
            for (int q = 0; q < G; ++q) ok = ok && (u >= units || ready4(v[i][q]));
        }
        if (ok || !poll_again(st, spin_limit, spins)) return;
        RetryUnits<0, NR, G, T>::run(src, base, units, v, tid);
    }
}

// src: the input (an op's own x, or the producer's copy for this launch);
// produced: whether to wait for sentinels.
template <int NR, int T = kStreamThreads>
__device__ inline void stage_requant(gcfloat src, bool produced, int k, uint32_t* st, int spin_limit,
                                     int4v* lds_q, float* lds_dx, int tid = (int)threadIdx.x) {
    const int units = k / 8;
    int spins = 0;
    for (int base = 0; base < units; base += NR * T) {
        float4v v[NR][2];
        issue_units<NR, 2, T>(src, base, units, v, tid);
        if (produced) await_units<NR, 2, T>(src, base, units, v, st, spin_limit, spins, tid);
        // units = 4 * blocks and T is a multiple of the wave, so the four
        // lanes of a block are in the same wave and all (in)active together
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = base + tid + i * T;
            if (u < units) requant_unit(v[i][0], v[i][1], u, lds_q, lds_dx);
        }
    }
}

template <int NR, int T = kStreamThreads>
__device__ inline void stage_f32(gcfloat src, bool produced, int k, uint32_t* st, int spin_limit, float4v* lds_x,
                                 int tid = (int)threadIdx.x) {
    const int units = k / 4;
    int spins = 0;
    for (int base = 0; base < units; base += NR * T) {
        float4v v[NR][1];
        issue_units<NR, 1, T>(src, base, units, v, tid);
        if (produced) await_units<NR, 1, T>(src, base, units, v, st, spin_limit, spins, tid);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = base + tid + i * T;
            if (u < units) lds_x[f32_slot(u)] = v[i][0];
        }
    }
}

// An op marked as depending on everything before it waits until the
// previous op's whole output is written in this launch (as a reader of that
// output would), re-reading the groups that still hold sentinels.
template <int T = kStreamThreads>
__device__ inline void wait_range(gcfloat p, int n, uint32_t* st, int spin_limit, int tid = (int)threadIdx.x) {
    const int units = n / 4;
    int spins = 0;
    for (int base = 0; base < units; base += 4 * T) {
        float4v v[4][1];
        issue_units<4, 1, T>(p, base, units, v, tid);
        await_units<4, 1, T>(p, base, units, v, st, spin_limit, spins, tid);
    }
    // the last n % 4 values, one per thread
    const int i = 4 * units + tid;
    if (i < n) {
        const gcu32 q = reinterpret_cast<gcu32>(p + i);
        while (__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == kSentinel &&
               poll_again(st, spin_limit, spins)) {
        }
    }
}

// The results of a workgroup's tiles of one op wait in LDS (res[tile][wave]:
// the wave's partial sum) until the op's end, so that the row loop issues
// no stores: on this GPU stores count against the same in-order counter as
// loads, and a store on some paths of the loop only would leave the
// compiler unable to tell how many weight loads are still in flight (it
// would then wait for all of them before every item).
// res[tile][group * S + part] holds the partial sum of that part of the
// group's row of the tile.
__device__ inline void keep_part(float acc, int j, int slot, float* lds_res) {
    if (threadIdx.x % kWave == 0) lds_res[j * kStreamWaves + slot] = acc;
}

// After the op's rows (and a barrier): the split-K partials meet in part
// order (the order of the eager kernels); every row is stored in y and in
// this launch's copy, and the next launch's copy is reset.
__device__ inline void flush_tiles(int tiles_wg, int grid, int n, int S, const float* lds_res, gfloat y,
                                   gfloat ynow, gfloat ynext) {
    constexpr int waves = kStreamWaves;
    const int groups = waves / S;
    for (int i = (int)threadIdx.x; i < tiles_wg * groups; i += kStreamThreads) {
        const int j = i / groups, grp = i % groups;
        const int row = ((int)blockIdx.x + j * grid) * groups + grp;
        if (row < n) {
            const float* part = lds_res + j * waves + grp * S;
            float total = part[0];
            for (int p = 1; p < S; ++p) total += part[p];
            y[row] = total;
            __hip_atomic_store(ynow + row, total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ynext + row, __uint_as_float(kSentinel), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Geometry of one op for this wave (wave-uniform).
struct OpGeom {
    gptr<uint8_t> w;
    gcfloat src;     // staged input: the op's x, or the producer's copy for this launch
    bool produced;   // src is a producer's copy (wait for sentinels)
    gfloat y;
    gfloat ynow, ynext;  // this op's copies: written now / reset for the next launch
    int n, k, S, C, NB, nl, sbl;
    int64_t row_bytes;
};

template <int WAVES>
__device__ inline OpGeom op_geom(const StreamOp& op, uint32_t parity) {
    OpGeom g;
    g.w = (gptr<uint8_t>)op.w;
    g.produced = op.xs != nullptr;
    g.src = g.produced ? (gcfloat)(op.xs + parity * op.xs_stride) : (gcfloat)op.x;
    g.y = (gfloat)op.y;
    g.ynow = (gfloat)(op.ys + parity * op.ys_stride);
    g.ynext = (gfloat)(op.ys + (parity ^ 1u) * op.ys_stride);
    g.n = op.n;
    g.k = op.k;
    g.S = op.split;
    g.C = (int)chunk_count(op.k);
    g.NB = op.k / kBlock;
    g.nl = g.NB - (g.C - 1) * kChunkBlocks;
    g.sbl = (int)scale_section_bytes(g.nl);
    g.row_bytes = packed_row_bytes(op.k);
    return g;
}

template <int WAVES, int U>
__device__ inline Sched op_sched(const OpGeom& g, int grid) {
    return Sched(g.C, g.S, U, WAVES, g.n, (g.n + WAVES / g.S - 1) / (WAVES / g.S), grid);
}

// A rotating-ring item of an op's matrix (see q8_load_rot).
struct OpRotLoad {
    const OpGeom* g;
    template <typename Regs>
    __device__ void operator()(Regs& R, const RotSched& rs, const RotCursor& it) const {
        q8_load_rot(R, g->w, g->row_bytes, g->nl, g->sbl, rs, it);
    }
};

// s_waitcnt immediate (gfx9 encoding): vector memory count 0, the export and
// LDS/scalar counts at their maxima (no wait).
constexpr int kWaitVmcnt0 = 0x0F70;

template <bool F32>
__device__ inline void stage(const OpGeom& g, uint8_t* smem, uint32_t* st, int spin_limit) {
    // one round trip for k up to 24576 (requantized) or 20480 (f32) at 16 waves
    if constexpr (F32) {
        stage_f32<5>(g.src, g.produced, g.k, st, spin_limit, reinterpret_cast<float4v*>(smem));
    } else {
        stage_requant<3>(g.src, g.produced, g.k, st, spin_limit, reinterpret_cast<int4v*>(smem),
                         reinterpret_cast<float*>(smem + (size_t)g.C * 2 * kWave * 16));
    }
}

template <int WAVES, int U, int N, bool F32>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(WAVES / 4)))
stream_kernel(const StreamOp* __restrict__ ops, int n_ops, uint32_t* __restrict__ st, int spin_limit) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ uint32_t parity_s;
    if (threadIdx.x == 0) {
        const uint64_t old = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(st + kStCounter), (uint64_t)1,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        parity_s = (uint32_t)(old / gridDim.x) & 1u;
    }
    __syncthreads();
    const uint32_t parity = parity_s;
    const int grid = (int)gridDim.x;

    Q8Regs<U> R[N];
    StreamOp op = ops[0];
    OpGeom g = op_geom<WAVES>(op, parity);
    Sched sc = op_sched<WAVES, U>(g, grid);
    const int wp = wave_id();  // slot in the group: wave % S (S divides 16)
    RotSched rs;
    rs.set(sc, wp);
    WSG_TL_OP(0, 2);
    rot_prologue(rs, R, OpRotLoad{&g});
    for (int j = 0;;) {
        if (op.dep) wait_range((gcfloat)(op.dep + parity * op.dep_stride), op.dep_n, st, spin_limit);
        stage<F32>(g, smem, st, spin_limit);
        // the staging has waited for every load before it (they complete in
        // order); saying so lets the compiler know it on every path, so the
        // row loop starts from a known count and its waits stay exact
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        WSG_TL_OP(j, 3);

        const size_t act_bytes = F32 ? lds_f32act_bytes(g.C) : lds_q8act_bytes(g.C);
        float* lds_res = reinterpret_cast<float*>(smem + act_bytes);
        const float4v* lds_x = reinterpret_cast<const float4v*>(smem);
        const int4v* lds_q = reinterpret_cast<const int4v*>(smem);
        const float* lds_dx = reinterpret_cast<const float*>(smem + (size_t)g.C * 2 * kWave * 16);
        auto compute = [&](const Q8Regs<U>& r, const Sched& s1, int row, int m, float& acc) {
            if constexpr (F32) {
                q8_f32_item<U>(r, s1, m, g.NB, lds_x, acc);
            } else {
                q8_i8_item<U, false>(r, s1, m, g.NB, lds_q, lds_dx, row, nullptr, acc);
            }
        };
        // parts this wave plays in no tile's chunks still meet as zeros
        if (threadIdx.x % kWave < (unsigned)sc.tiles_wg) {
            const int t = (int)(threadIdx.x % kWave);
            if (rs.items(t) == 0) lds_res[t * kStreamWaves + sc.group * sc.S + rs.part(t)] = 0.0f;
        }
        rot_loop(rs, R, OpRotLoad{&g}, compute, [&](float acc, int t, int slot) { keep_part(acc, t, slot, lds_res); });
        __syncthreads();  // every tile's partial sums are in LDS; the activation is dead
        WSG_TL_OP(j, 4);
        flush_tiles(sc.tiles_wg, grid, g.n, g.S, lds_res, g.y, g.ynow, g.ynext);
        WSG_TL_OP(j, 5);
        if (++j == n_ops) break;

        op = ops[j];
        g = op_geom<WAVES>(op, parity);
        sc = op_sched<WAVES, U>(g, grid);
        rs.set(sc, wp);
        WSG_TL_OP(j, 2);
        rot_prologue(rs, R, OpRotLoad{&g});
    }
}

template <bool F32>
const void* stream_kernel_ptr() {
    return reinterpret_cast<const void*>(stream_kernel<kStreamWaves, kStreamUnroll, kStreamSets, F32>);
}


}  // namespace

size_t stream_state_bytes() { return (size_t)kStWords * sizeof(uint32_t); }
size_t stream_error_word() { return kStError; }
size_t stream_detail_word() { return kStDetail; }

int stream_config(int max_k, bool f32, int* waves, int* grid, size_t* lds) {
    const void* kern = f32 ? stream_kernel_ptr<true>() : stream_kernel_ptr<false>();
    const int C = (int)chunk_count(max_k);
    const size_t act = f32 ? lds_f32act_bytes(C) : lds_q8act_bytes(C);
    const size_t bytes = act + (size_t)kMaxTiles * kStreamWaves * sizeof(float);
    if (bytes > 65536) (void)hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kStreamWaves * kWave, bytes) != hipSuccess ||
        per_cu < 1)
        return WSG_ERR_HIP;
    // one workgroup per CU (the grid never exceeds what is co-resident)
    *waves = kStreamWaves;
    *grid = device_info().cus;
    *lds = bytes;
    return WSG_OK;
}

int stream_launch(const StreamOp* ops_dev, int n_ops, bool f32, uint32_t* state_dev, int grid, size_t lds,
                  int spin_limit, hipStream_t stream) {
    const void* kern = f32 ? stream_kernel_ptr<true>() : stream_kernel_ptr<false>();
    void* args[] = {&ops_dev, &n_ops, &state_dev, &spin_limit};
    (void)hipLaunchKernel(kern, dim3(grid), dim3(kStreamWaves * kWave), args, lds, stream);
    return launch_status();
}

int stream_split(bool f32, int64_t n, int64_t k) { return gemv_split(f32, n, k); }

void stream_shape(int* waves, int* unroll, int* sets) {
    *waves = kStreamWaves;
    *unroll = kStreamUnroll;
    *sets = kStreamSets;
}

int64_t stream_max_rows(int split, int grid) { return (int64_t)kMaxTiles * grid * (kStreamWaves / split); }

#ifdef WSG_TIMELINE
int stream_timeline_set(void* buf, uint32_t modulus) { return tl_set_here(buf, modulus); }
#endif

}  // namespace wsg
