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
constexpr int kSiteFreeSlot = 2, kSiteFullSlot = 3, kSiteConsumers = 4;  // the LDS-ring handshakes
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
            if (u < units) lds_x[StageF32<1>::slot(u)] = v[i][0];
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
    const int wp = (int)(threadIdx.x / kWave);  // slot in the group: wave % S (S divides 16)
    RotSched rs;
    rs.set(sc, wp);
    rot_prologue(rs, R, OpRotLoad{&g});
    for (int j = 0;;) {
        if (op.dep) wait_range((gcfloat)(op.dep + parity * op.dep_stride), op.dep_n, st, spin_limit);
        stage<F32>(g, smem, st, spin_limit);
        // the staging has waited for every load before it (they complete in
        // order); saying so lets the compiler know it on every path, so the
        // row loop starts from a known count and its waits stay exact
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();

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
        flush_tiles(sc.tiles_wg, grid, g.n, g.S, lds_res, g.y, g.ynow, g.ynext);
        if (++j == n_ops) break;

        op = ops[j];
        g = op_geom<WAVES>(op, parity);
        sc = op_sched<WAVES, U>(g, grid);
        rs.set(sc, wp);
        rot_prologue(rs, R, OpRotLoad{&g});
    }
}

template <bool F32>
const void* stream_kernel_ptr() {
    return reinterpret_cast<const void*>(stream_kernel<kStreamWaves, kStreamUnroll, kStreamSets, F32>);
}


// ------------------------------------------------------------------------
// LDS-ring token kernel: the weight stream decoupled from the chain's data
// dependencies.  In the kernel above every wave both streams weights and
// waits for its next input, and a wave's loads complete in order, so the
// input staging at each GEMV start waits behind every weight load issued
// before it: at most three items per wave can be requested ahead, and HBM
// idles for the rest of each dependency wait (~4-5 us at each of the 256
// GEMV boundaries of a 27B token).  Here each 16-wave workgroup splits into
// P producer waves and 16 - P consumer waves.  Producers only copy weights
// from HBM into a ring of LDS slots with gfx950's direct-to-LDS loads
// (global_load_lds: no registers, 16 bytes per lane), one slot per item of
// one 2048-weight chunk of one row, in the order the workgroup's rows and
// chunks are consumed, GEMV after GEMV: they never wait for an activation,
// only for a free slot.  Consumers stage each GEMV's input (requantized
// into one of two LDS buffers, so staging the next input does not wait for
// the current rows), then take the workgroup's rows in turn (rows of all
// GEMVs dealt round-robin), read each item from its slot, free the slot
// and store each row as soon as it is done.  While consumers wait for an
// input, producers keep filling the ring (~120 KB, ~5 us of this CU's
// share of HBM), so the stream runs on through the wait.
//
// Slot handshakes live in LDS: full[slot] = the item number a producer
// published there, freed[slot] = the last item a consumer took out of it.
// A producer publishes an item once the vector memory counter shows its
// loads done (the counter counts the LDS writes of these loads; each
// producer keeps D items in flight and waits with a constant count).  The
// producers access the flags through inline assembly: the compiler cannot
// tell the flags from the DMA'd slots and would otherwise wait for every
// load in flight before each flag access.  Each wave's LDS operations
// complete in order, which orders data before flag and read before release.
// Each row is reduced by one wave in chunk order and a butterfly, as the
// unsplit eager kernel reduces it.  Every wait is bounded as in the kernel
// above.

__device__ inline uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ inline void lds_put(uint32_t a, int v) { asm volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(v) : "memory"); }
__device__ inline void lds_inc(uint32_t a, int v) { asm volatile("ds_add_u32 %0, %1" ::"v"(a), "v"(v) : "memory"); }
__device__ inline int lds_get(uint32_t a) {
    int v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
    return v;
}

// Rows of an op this workgroup owns: blockIdx.x + i * grid.
__device__ inline int ring_rows(int n, int grid) {
    return (int)blockIdx.x < n ? (n - 1 - (int)blockIdx.x) / grid + 1 : 0;
}

// Item s of the workgroup's sequence (op after op; within an op, row
// i = e / C and chunk e % C of its e-th item) is fetched by producer wave
// s % P into its own sub-ring of NSp slots: slot ring_slot(s).  A slot is
// the chunk's device layout reordered: [first 16 codes of 64 blocks][last
// 16 codes][64 fp16 scales] (2176 bytes).
template <int P>
__device__ inline int ring_slot(int s, int NSp) {
    return (s % P) * NSp + (s / P) % NSp;
}

// D consecutive flags of a sub-ring (16-byte aligned), in one LDS round trip.
template <int D>
__device__ inline void lds_get_flags(uint32_t a, int (&f)[D]) {
    static_assert(D == 4 || D == 8 || D == 12, "flag batches of 4, 8 or 12");
    int4v x0, x1, x2;
    if constexpr (D == 4) {
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x0) : "v"(a) : "memory");
    } else if constexpr (D == 8) {
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(x0), "=&v"(x1)
                     : "v"(a)
                     : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %3\n\tds_read_b128 %1, %3 offset:16\n\tds_read_b128 %2, %3 offset:32\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(x0), "=&v"(x1), "=&v"(x2)
            : "v"(a)
            : "memory");
    }
    const int4v xs[3] = {x0, x1, x2};
#pragma unroll
    for (int b = 0; b < D; ++b) f[b] = xs[b / 4][b % 4];
}

// The op of the item a producer requests next (wave-uniform: the
// descriptors are read with scalar loads, which do not count against the
// vector memory counter the weight ring relies on).
struct ProdCursor {
    int j = -1, op_base = 0, items_j = 0, C = 1, nl = 0, sbl = 0;
    int64_t row_bytes = 0;
    gptr<uint8_t> w = nullptr;
    __device__ void seek(const StreamOp* __restrict__ ops, int s, int grid) {
        while (s - op_base >= items_j) {
            op_base += items_j;
            j = __builtin_amdgcn_readfirstlane(j + 1);
            const StreamOp* op = ops + j;
            const int kk = __builtin_amdgcn_readfirstlane(op->k);
            C = (int)chunk_count(kk);
            nl = kk / kBlock - (C - 1) * kChunkBlocks;
            sbl = (int)scale_section_bytes(nl);
            row_bytes = packed_row_bytes(kk);
            const uint64_t wa = reinterpret_cast<uint64_t>(op->w);
            w = (gptr<uint8_t>)((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)wa) |
                                ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(wa >> 32)) << 32));
            items_j = ring_rows(__builtin_amdgcn_readfirstlane(op->n), grid) * C;
        }
    }
};

// Producer wave p fetches its items s = k P + p (k = 0, 1, ...) through a
// ring of R register sets, as the row loops of the other kernels do: every
// step writes the oldest set into its LDS slot, publishes it and refills
// the set with the item R further on (past the workgroup's items: the idle
// region), so R - 1 items stay in flight and the compiler waits for exactly
// one set at a time.  Before the first item of each batch of D sub-slots it
// checks, in one LDS round trip, that the batch's slots are free (their
// items NSp earlier consumed).
template <int P, int R>
__device__ __attribute__((always_inline)) inline void ring_produce(const StreamOp* __restrict__ ops, int n_ops, int grid, uint8_t* ring, int NSp,
                                    uint32_t full_a, uint32_t freed_a, uint32_t* st, int spin_limit) {
    constexpr int D = 4;
    const int p = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int lane = (int)threadIdx.x % kWave;
    int total = 0;  // items of this workgroup
    for (int j = 0; j < n_ops; ++j) total += ring_rows(ops[j].n, grid) * (int)chunk_count(ops[j].k);
    const int mine = total > p ? (total - 1 - p) / P + 1 : 0;  // this wave's items
    const uint32_t my_full = full_a + 4u * (uint32_t)(p * NSp);
    const uint32_t my_freed = freed_a + 4u * (uint32_t)(p * NSp);
    uint8_t* my_ring = ring + (size_t)(p * NSp) * kFullChunkBytes;

    ProdCursor cur;
    // requests item k of this wave (the idle region past its last item)
    auto load = [&](Q8Regs<1>& r, int k) {
        gptr<uint8_t> cp = idle_bytes();
        int nbc = kChunkBlocks, sb = 2 * kChunkBlocks;
        if (k < mine) {
            const int s = k * P + p;
            cur.seek(ops, s, grid);
            const int e = s - cur.op_base;
            const int i = e / cur.C, c = e - i * cur.C;
            const int row = (int)blockIdx.x + i * grid;
            const bool last = c == cur.C - 1;
            nbc = last ? cur.nl : kChunkBlocks;
            sb = last ? cur.sbl : 2 * kChunkBlocks;
            cp = cur.w + (int64_t)row * cur.row_bytes + (int64_t)c * kFullChunkBytes;
        }
        const int l = lane < nbc ? lane : nbc - 1;  // past a ragged chunk: re-read its last block
        r.sc[0] = load_u16<true>(cp + 2 * l);
        r.a[0] = load16<true>(cp + sb + 16 * l);
        r.b[0] = load16<true>(cp + sb + 16 * nbc + 16 * l);
    };
    bool failed = false;
    // writes item k (landed in r) into its slot and publishes it
    auto store = [&](const Q8Regs<1>& r, int k) {
        if (failed || k >= mine) return;
        const int sub = k % NSp;
        if (k % D == 0) {  // the batch's slots must be free
            int spins = 0;
            for (;;) {
                int f[D];
                lds_get_flags<D>(my_freed + 4u * (uint32_t)sub, f);
                int bad = -1;
#pragma unroll
                for (int b = 0; b < D; ++b) {
                    const int s = (k + b) * P + p;
                    if (k + b < mine && f[b] < s - P * NSp) bad = b;
                }
                if (bad < 0) break;
                if (!poll_again(st, spin_limit, spins, kSiteFreeSlot, cur.j, (k + bad) * P + p - P * NSp, f[bad])) {
                    failed = true;
                    return;
                }
            }
        }
        uint8_t* it = my_ring + (size_t)sub * kFullChunkBytes;
        reinterpret_cast<int4v*>(it)[lane] = r.a[0];
        reinterpret_cast<int4v*>(it + 16 * kWave)[lane] = r.b[0];
        reinterpret_cast<uint16_t*>(it + 32 * kWave)[lane] = r.sc[0];
        if (lane == 0) lds_put(my_full + 4u * (uint32_t)sub, k * P + p);  // after the data (LDS order)
    };

    Q8Regs<1> regs[R];
#pragma unroll
    for (int r = 0; r < R; ++r) load(regs[r], r);
    for (int k0 = 0; k0 < mine; k0 += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            store(regs[r], k0 + r);
            load(regs[r], k0 + r + R);
        }
    }
    // the last refills read the idle region: let them land before the wave ends
#pragma unroll
    for (int r = 0; r < R; ++r) opaque(regs[r].a[0]), opaque(regs[r].b[0]);
}

// Consumer waves: per op, stage the input into act buffer j % 2, meet at an
// LDS counter, then take rows t_base + i (the op's i-th row of this
// workgroup) with (t_base + i) % NC == this wave.
template <int W, int P>
__device__ __attribute__((always_inline)) inline void ring_consume(const StreamOp* __restrict__ ops, int n_ops, int grid, uint32_t parity,
                                    uint8_t* smem, int act_bytes, const uint8_t* ring, int NSp, uint32_t full_a,
                                    uint32_t freed_a, uint32_t bar_a, uint32_t* st, int spin_limit) {
    constexpr int NC = W - P;
    constexpr int T = NC * kWave;
    // rounds of staging loads in flight: a 17408-value input in one round trip
    constexpr int NR = (17408 / 8 + T - 1) / T;
    const int tid = (int)threadIdx.x - P * kWave;
    const int cw = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = (int)threadIdx.x % kWave;
    int s_base = 0, t_base = 0;
    for (int j = 0; j < n_ops; ++j) {
        const StreamOp& op = ops[j];
        const OpGeom g = op_geom<W>(op, parity);
        const int rows = ring_rows(g.n, grid);
        uint8_t* act = smem + (size_t)(j & 1) * act_bytes;
        const int4v* lds_q = reinterpret_cast<const int4v*>(act);
        const float* lds_dx = reinterpret_cast<const float*>(act + (size_t)g.C * 2 * kWave * 16);
        if (op.dep) wait_range<T>((gcfloat)(op.dep + parity * op.dep_stride), op.dep_n, st, spin_limit, tid);
        stage_requant<NR, T>(g.src, g.produced, g.k, st, spin_limit, reinterpret_cast<int4v*>(act),
                            reinterpret_cast<float*>(act + (size_t)g.C * 2 * kWave * 16), tid);
        // every consumer wave has staged its share (and so finished op j - 1)
        if (lane == 0) lds_inc(bar_a, 1);
        {
            int spins = 0;
            int seen;
            while ((seen = lds_get(bar_a)) < NC * (j + 1))
                if (!poll_again(st, spin_limit, spins, kSiteConsumers, j, NC * (j + 1), seen)) return;
        }
        int i = cw - t_base % NC;
        if (i < 0) i += NC;
        for (; i < rows; i += NC) {
            const int row = (int)blockIdx.x + i * grid;
            int s = s_base + i * g.C;
            float acc = 0.0f;
            for (int c = 0; c < g.C; ++c, ++s) {
                const int slot = ring_slot<P>(s, NSp);
                int spins = 0;
                int seen;
                while ((seen = lds_get(full_a + 4 * slot)) != s)
                    if (!poll_again(st, spin_limit, spins, kSiteFullSlot, j, s, seen)) return;
                const uint8_t* it = ring + (size_t)slot * kFullChunkBytes;
                const int blk = c * kWave + lane;
                if (blk < g.NB) {
                    const int4v wa = reinterpret_cast<const int4v*>(it)[lane];
                    const int4v wb = reinterpret_cast<const int4v*>(it + 16 * kWave)[lane];
                    const uint16_t sc = reinterpret_cast<const uint16_t*>(it + 32 * kWave)[lane];
                    const int4v xa = lds_q[(c * 2 + 0) * kWave + lane];
                    const int4v xb = lds_q[(c * 2 + 1) * kWave + lane];
                    int d = 0;
                    d = __builtin_amdgcn_sdot4(wa.x, xa.x, d, false);
                    d = __builtin_amdgcn_sdot4(wa.y, xa.y, d, false);
                    d = __builtin_amdgcn_sdot4(wa.z, xa.z, d, false);
                    d = __builtin_amdgcn_sdot4(wa.w, xa.w, d, false);
                    d = __builtin_amdgcn_sdot4(wb.x, xb.x, d, false);
                    d = __builtin_amdgcn_sdot4(wb.y, xb.y, d, false);
                    d = __builtin_amdgcn_sdot4(wb.z, xb.z, d, false);
                    d = __builtin_amdgcn_sdot4(wb.w, xb.w, d, false);
                    const float t = half_bits_to_float(sc) * lds_dx[blk];
                    acc = __builtin_fmaf(t, (float)d, acc);
                }
                if (lane == 0) lds_put(freed_a + 4 * slot, s);  // after this wave's reads of the slot
            }
            acc = wave_sum(acc);
            if (lane == 0) {
                g.y[row] = acc;
                __hip_atomic_store(g.ynow + row, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(g.ynext + row, __uint_as_float(kSentinel), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        s_base += rows * g.C;
        t_base += rows;
    }
}

// LDS: [act 0][act 1][ring NS x 2176][full NS][freed NS][barrier, parity],
// NS = P NSp (a sub-ring of NSp slots per producer).
template <int W, int P, int R>
__global__ void __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(W / 4)))
ring_kernel(const StreamOp* __restrict__ ops, int n_ops, uint32_t* __restrict__ st, int spin_limit, int act_bytes,
            int NSp) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int NS = P * NSp;
    uint8_t* ring = smem + 2 * (size_t)act_bytes;
    int* full = reinterpret_cast<int*>(ring + (size_t)NS * kFullChunkBytes);
    int* freed = full + NS;
    int* misc = freed + NS;
    // slot i of sub-ring q first holds item s = (i - q NSp) P + q: as if its
    // item s - P NSp had been consumed
    for (int i = (int)threadIdx.x; i < NS; i += W * kWave) {
        const int q = i / NSp;
        full[i] = -1;
        freed[i] = (i - q * NSp) * P + q - P * NSp;
    }
    if (threadIdx.x == 0) {
        misc[0] = 0;
        const uint64_t old = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(st + kStCounter), (uint64_t)1,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        misc[1] = (int)((old / gridDim.x) & 1u);
    }
    __syncthreads();
    const uint32_t parity = (uint32_t)misc[1];
    const int grid = (int)gridDim.x;
    if ((int)threadIdx.x < P * kWave) {
        ring_produce<P, R>(ops, n_ops, grid, ring, NSp, lds_offset(full), lds_offset(freed), st, spin_limit);
    } else {
        ring_consume<W, P>(ops, n_ops, grid, parity, smem, act_bytes, ring, NSp, lds_offset(full), lds_offset(freed),
                        lds_offset(misc), st, spin_limit);
    }
}

// Shapes of the ring kernel: waves per workgroup (fewer waves leave more
// registers per wave), producer waves and the register sets each keeps
// (R - 1 items in flight).  Variant 0 is the default.
struct RingVariant {
    int waves, producers, depth;
    const void* kern;
};
constexpr int kRingVariants = 2;
const RingVariant* ring_variant(int variant) {
    // (16 waves: at most 128 registers each.  Shapes of 8 and 12 waves,
    // whose producers can hold 16-21 items, measured slower and keep
    // their staging in scratch memory.)
    static const RingVariant v[kRingVariants] = {
        {16, 4, 8, reinterpret_cast<const void*>(ring_kernel<16, 4, 8>)},
        {16, 2, 10, reinterpret_cast<const void*>(ring_kernel<16, 2, 10>)},
    };
    return variant >= 0 && variant < kRingVariants ? &v[variant] : nullptr;
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

int ring_config(int max_k, int variant, int* grid, size_t* lds, int* act_bytes, int* slots) {
    const RingVariant* v = ring_variant(variant);
    if (!v) return WSG_ERR_MODE;
    const int C = (int)chunk_count(max_k);
    const int act = (int)lds_q8act_bytes(C);
    const int64_t fixed = 2 * (int64_t)act + 16;
    // each producer's sub-ring: a whole number of 4-slot batches (a batch's
    // slots hold items that have all been written and published before it)
    const int64_t per = ((int64_t)device_info().max_lds - fixed) / (kFullChunkBytes + 8) / v->producers;
    const int64_t nsp = per / 4 * 4;
    if (nsp < 4) return WSG_ERR_SHAPE;
    const int64_t ns = nsp * v->producers;
    const size_t bytes = (size_t)(fixed + ns * (kFullChunkBytes + 8));
    if (hipFuncSetAttribute(v->kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
        return WSG_ERR_HIP;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, v->kern, v->waves * kWave, bytes) != hipSuccess ||
        per_cu < 1)
        return WSG_ERR_HIP;
    *grid = device_info().cus;  // one workgroup per CU: every producer of a consumer's input is resident
    *lds = bytes;
    *act_bytes = act;
    *slots = (int)nsp;
    return WSG_OK;
}

int ring_shape(int variant, int* waves, int* producers, int* depth) {
    const RingVariant* v = ring_variant(variant);
    if (!v) return WSG_ERR_MODE;
    *waves = v->waves;
    *producers = v->producers;
    *depth = v->depth;
    return WSG_OK;
}

int ring_variants() { return kRingVariants; }

int ring_launch(const StreamOp* ops_dev, int n_ops, int variant, uint32_t* state_dev, int grid, size_t lds,
                int act_bytes, int slots, int spin_limit, hipStream_t stream) {
    const RingVariant* v = ring_variant(variant);
    if (!v) return WSG_ERR_MODE;
    void* args[] = {&ops_dev, &n_ops, &state_dev, &spin_limit, &act_bytes, &slots};
    (void)hipLaunchKernel(v->kern, dim3(grid), dim3(v->waves * kWave), args, lds, stream);
    return launch_status();
}

}  // namespace wsg
