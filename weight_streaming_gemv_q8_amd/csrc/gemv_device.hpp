// Device building blocks of the GEMV kernels (gfx950, wave64): the work
// schedule, the pipelined row loop, weight-item loads, activation staging in
// LDS and the per-item dot products.  Included by gemv.hip and stream.hip;
// everything here is internal to each translation unit.
#pragma once

#include "common.hpp"

namespace wsg {
namespace {

constexpr int kActQ8 = 0, kActF32 = 1, kActRequant = 2;  // = WSG_ACT_*

// ------------------------------------------------------------------ LDS
// Layouts of the staged activation (per 2048-weight chunk c, lane l):
//  int8 paths : int4v q[C][2][64]   (half h of block 64c+l), float dx[C*64]
//  f32 path   : float4v x[C][8][64] (values 4g..4g+3 of block 64c+l)
//  bf16 path  : float4v x[C'][2][2][64] over 1024-element chunks:
//               values 1024c + 512h + 8l + 4j .. +3

__host__ __device__ inline size_t lds_q8act_bytes(int C) { return (size_t)C * (2 * kWave * 16 + kWave * 4); }
__host__ __device__ inline size_t lds_f32act_bytes(int C) { return (size_t)C * 8 * kWave * 16; }
__host__ __device__ inline int bf16_chunks(int k) { return (k + 1023) / 1024; }
__host__ __device__ inline size_t lds_bf16_bytes(int k) { return (size_t)bf16_chunks(k) * 4 * kWave * 16; }
// tail of the LDS allocation: S partial sums per tile and the argmax keys
template <int WAVES>
__host__ __device__ constexpr size_t lds_tail_bytes() {
    return WAVES * sizeof(float) + WAVES * sizeof(uint64_t) + 16;
}

// --------------------------------------------------------- work schedule
// A workgroup walks row tiles t = blockIdx.x + j * gridDim.x.  Wave w owns
// row t * GROUPS + w / S of each tile and the chunks c = p, p + S, ... of it
// (p = w % S).  Its work is a flat sequence of items (tile j, item m); item m
// covers U of its chunks.  Loads of item i+1 are issued before item i is
// consumed, and the loads of the first item before the activation staging
// completes, so HBM sees requests from the first cycles of the launch.
struct Sched {
    int C, S, U, part, group, groups, n, tiles_wg, ipt, grid;
    __device__ Sched(int C_, int S_, int U_, int waves, int n_, int tiles)
        : Sched(C_, S_, U_, waves, n_, tiles, (int)gridDim.x) {}
    // grid: the number of workgroups (gridDim.x), when the caller has it at hand
    __device__ Sched(int C_, int S_, int U_, int waves, int n_, int tiles, int grid_) {
        grid = grid_;
        C = C_;
        S = S_;
        U = U_;
        const int wave = wave_id();
        part = wave % S;
        group = wave / S;
        groups = waves / S;
        n = n_;
        tiles_wg = blockIdx.x < (unsigned)tiles ? (tiles - 1 - (int)blockIdx.x) / grid + 1 : 0;
        const int count = part < C ? (C - part + S - 1) / S : 0;
        ipt = (count + U - 1) / U;
    }
    __device__ int row(int j) const { return ((int)blockIdx.x + j * grid) * groups + group; }
    // chunk of slot u in item m
    __device__ int chunk(int m, int u) const { return part + S * (m * U + u); }
};

// Epilogue shared by all paths: combine split-K partials in part order,
// then store y (and/or fold the row into the workgroup's argmax key).
template <int WAVES, int S, bool ARGMAX>
__device__ inline void finish_row(float acc, int row, int n, int lane, int wave, float* lds_part, float* y,
                                  uint64_t& best) {
    const int part = wave % S;
    float total = acc;
    if constexpr (S > 1) {
        if (lane == 0) lds_part[wave] = acc;
        __syncthreads();
        if (part == 0) {
            total = lds_part[wave];
#pragma unroll
            for (int p = 1; p < S; ++p) total += lds_part[wave + p];
        }
        __syncthreads();
    }
    if (part == 0 && row < n) {
        if constexpr (ARGMAX) {
            const uint64_t key = argmax_key(total, (uint32_t)row);
            best = key > best ? key : best;
            if (y != nullptr && lane == 0) y[row] = total;
        } else {
            if (lane == 0) y[row] = total;
        }
    }
}

template <int WAVES>
__device__ inline void write_block_key(uint64_t best, int lane, int wave, uint64_t* lds_key, uint64_t* keys) {
    if (lane == 0) lds_key[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t m = lds_key[0];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) m = lds_key[w] > m ? lds_key[w] : m;
        keys[blockIdx.x] = m;
    }
}

// Weight loads with nothing to fetch (past a wave's items, past the matrix,
// past a row's chunks) read this small region instead, which stays in the
// L2 cache.  So every path through a row loop issues the same loads, and the
// compiler, which tracks loads in flight per program point, can wait for
// exactly one ring set at a time; a load issued on some paths only would
// make it wait for every outstanding load before each item.
__device__ __align__(256) uint8_t g_idle[4096];
__device__ inline gptr<uint8_t> idle_bytes() { return (gptr<uint8_t>)(const uint8_t*)g_idle; }

// Item i of a wave's schedule is (tile i / ipt, item i % ipt).
struct ItemCursor {
    int j = 0, m = 0;
    __device__ void next(int ipt) {
        if (++m == ipt) {
            m = 0;
            ++j;
        }
    }
};

// The pipelined row loop shared by all paths: a ring of N register sets
// holding items of weights.  A wave's T items are laid out at positions
// pad .. P-1 of a sequence of P = T rounded up to a multiple of N positions
// (the first pad = P - T positions hold nothing), position q in set q % N.
// ring_prologue() requests positions 0 .. N-1 (the caller issues it before
// the activation staging completes, so HBM sees requests from the first
// cycles; the empty positions read the idle region).  Each step of the main
// loop consumes position q and refills its set with position q + N, which
// always exists, so every step issues one item's loads and N - 1 items stay
// in flight while one is consumed; the last N positions are consumed
// without refills, so no load is left in flight at the end.  No loaded
// register is ever copied (a copy would force a wait for its load; the ring
// is unrolled, so every set index is a constant).  load(regs, item) issues
// an item's loads; compute(regs, row, m, acc) consumes it; finish(acc, j,
// row, valid) ends tile j (every wave calls it once per tile, as split-K
// needs).
struct Ring {
    int total, pad, groups;  // items, empty leading positions, groups of N positions
    template <int N>
    __device__ static Ring of(const Sched& sc) {
        Ring r;
        r.total = sc.ipt == 0 ? 0 : sc.tiles_wg * sc.ipt;
        const int P = (r.total + N - 1) / N * N;
        r.pad = P - r.total;
        r.groups = P / N;
        return r;
    }
};

// The item at position q of the ring (q >= pad), or past the schedule.
__device__ inline ItemCursor ring_item(const Sched& sc, const Ring& rg, int q) {
    ItemCursor it;
    const int i = q - rg.pad;
    if (i < 0 || sc.ipt == 0) {
        it.j = sc.tiles_wg;  // nothing: reads the idle region
    } else {
        it.j = i / sc.ipt;
        it.m = i - it.j * sc.ipt;
    }
    return it;
}

template <int N, typename Regs, typename LoadF>
__device__ inline void ring_prologue(const Sched& sc, Regs (&R)[N], LoadF&& load) {
    const Ring rg = Ring::of<N>(sc);
#pragma unroll
    for (int s = 0; s < N; ++s) load(R[s], ring_item(sc, rg, s));
}

template <int N, typename Regs, typename LoadF, typename ComputeF, typename FinishF>
__device__ inline void ring_loop(const Sched& sc, Regs (&R)[N], LoadF&& load, ComputeF&& compute,
                                 FinishF&& finish) {
    const Ring rg = Ring::of<N>(sc);
    if (rg.total == 0) {
        for (int j = 0; j < sc.tiles_wg; ++j) finish(0.0f, j, sc.row(j), false);
        return;
    }
    ItemCursor cur;                             // the next item to consume
    ItemCursor nxt = ring_item(sc, rg, N);      // the next item to request
    float acc = 0.0f;
    auto consume = [&](Regs& r, int q) {
        if (q < rg.pad) return;
        const int row = sc.row(cur.j);
        const bool valid = row < sc.n;
        if (valid) compute(r, row, cur.m, acc);
        if (cur.m == sc.ipt - 1) {
            if (valid) acc = wave_sum(acc);
            finish(acc, cur.j, row, valid);
            acc = 0.0f;
        }
        cur.next(sc.ipt);
    };
    for (int g = 0; g + 1 < rg.groups; ++g) {
#pragma unroll
        for (int s = 0; s < N; ++s) {
            consume(R[s], g * N + s);
            load(R[s], nxt);
            nxt.next(sc.ipt);
        }
    }
    const int q0 = (rg.groups - 1) * N;
#pragma unroll
    for (int s = 0; s < N; ++s) consume(R[s], q0 + s);
}

// ------------------------------------------------------ Q8_0 weight items
template <int U>
struct Q8Regs {
    int4v a[U], b[U];
    uint16_t sc[U];
};

// Requests item `it` of the wave's schedule: U chunks of one row, 3U loads
// whether or not the item, the row or a chunk exists (those read the idle
// region).  Lanes past a ragged chunk's last block re-read its last block
// (the same cache lines), so the loads are not divergent; compute skips
// them.
template <int U>
__device__ inline void q8_load_item(Q8Regs<U>& r, gptr<uint8_t> W, int64_t row_bytes, const Sched& sc, int nl,
                                    int sbl, const ItemCursor& it) {
    const int lane = threadIdx.x % kWave;
    const int row = it.j < sc.tiles_wg ? sc.row(it.j) : sc.n;
    const bool has_row = row < sc.n;
    const gptr<uint8_t> rowp = W + (int64_t)(has_row ? row : 0) * row_bytes;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = sc.chunk(it.m, u);
        const bool real = has_row && c < sc.C;
        const bool last = (c == sc.C - 1);
        const int nbc = last ? nl : kChunkBlocks;
        const int sb = last ? sbl : 2 * kChunkBlocks;
        // a wave-uniform item base plus a 32-bit per-lane offset: a scalar
        // base register and a vector offset in each load
        const uint32_t l = (uint32_t)(lane < nbc ? lane : nbc - 1);
        const gptr<uint8_t> cp = real ? rowp + (int64_t)c * kFullChunkBytes : idle_bytes();
        r.sc[u] = load_u16<true>(cp + 2u * l);
        r.a[u] = load16<true>(cp + ((uint32_t)sb + 16u * l));
        r.b[u] = load16<true>(cp + ((uint32_t)(sb + 16 * nbc) + 16u * l));
    }
}

// ------------------------------------------------------- rotating parts
// With split-K (S > 1) a row's chunks are dealt to S parts (part p takes
// chunks p, p + S, ...), and when the chunks do not divide evenly the low
// parts take more (the 27B down projection: 3, 2, 2, 2 chunks).  A wave
// that played part 0 in every tile would do half as much again as the
// others and hold up the workgroup at the end, so the wave of group slot w
// plays part (w + tile) % S: the heavy part passes round the waves.  Each
// part's partial sum is the same computation whichever wave makes it, and
// the parts still meet in part order, so the result depends neither on the
// rotation nor on the loop (ring_loop computes the same partials).
// One-chunk items (U = 1).
struct RotSched {
    const Sched* sc;
    int wp;          // this wave's slot within its group (its part in tile 0)
    int base, rem;   // part p takes base + (p < rem) chunks (S is a power of two)
    __device__ void set(const Sched& s, int slot) {
        sc = &s;
        wp = slot & (s.S - 1);
        base = s.C >> __builtin_ctz(s.S);
        rem = s.C & (s.S - 1);
    }
    __device__ int part(int j) const { return (wp + j) & (sc->S - 1); }
    __device__ int items_of(int p) const { return base + (p < rem ? 1 : 0); }
    __device__ int items(int j) const { return items_of(part(j)); }
    // the wave's items over all its tiles
    __device__ int total() const {
        int t = 0;
        for (int p = 0; p < sc->S; ++p) {
            const int j0 = (p - wp) & (sc->S - 1);
            if (j0 < sc->tiles_wg) t += ((sc->tiles_wg - 1 - j0) >> __builtin_ctz(sc->S)) * items_of(p) + items_of(p);
        }
        return t;
    }
};

// Walks a wave's items in order: (tile j, item m of that tile, its part p
// and item count); j reaches tiles_wg past the last item.
struct RotCursor {
    int j = 0, m = 0, p = 0, ipt = 0;
    __device__ void start(const RotSched& rs) {
        j = 0;
        m = 0;
        p = rs.wp;
        ipt = rs.items_of(p);
        if (ipt == 0) skip_empty(rs);
    }
    __device__ void skip_empty(const RotSched& rs) {  // only when a part has no chunks (C < S)
        while (j < rs.sc->tiles_wg && ipt == 0) {
            ++j;
            p = (p + 1) & (rs.sc->S - 1);
            ipt = rs.items_of(p);
        }
    }
    __device__ void next(const RotSched& rs) {
        if (++m == ipt) {
            m = 0;
            ++j;
            p = (p + 1) & (rs.sc->S - 1);
            ipt = rs.items_of(p);
            if (ipt == 0) skip_empty(rs);
        }
    }
};

// One item: chunk part(j) + S * m of the group's row of tile j (3 loads;
// the idle region past the wave's items or the matrix, see q8_load_item).
__device__ inline void q8_load_rot(Q8Regs<1>& R, gptr<uint8_t> W, int64_t row_bytes, int nl, int sbl,
                                   const RotSched& rs, const RotCursor& it) {
    const Sched& sc = *rs.sc;
    const int lane = threadIdx.x % kWave;
    const bool has_item = it.j < sc.tiles_wg;
    const int row = has_item ? sc.row(it.j) : sc.n;
    const bool has_row = row < sc.n;
    const int c = has_item ? it.p + sc.S * it.m : sc.C;
    const bool real = has_row && c < sc.C;
    const bool last = (c == sc.C - 1);
    const int nbc = last ? nl : kChunkBlocks;
    const int sb = last ? sbl : 2 * kChunkBlocks;
    const int l = lane < nbc ? lane : nbc - 1;
    const gptr<uint8_t> cp = real ? W + (int64_t)row * row_bytes + (int64_t)c * kFullChunkBytes : idle_bytes();
    R.sc[0] = load_u16<true>(cp + 2u * (uint32_t)l);
    R.a[0] = load16<true>(cp + ((uint32_t)sb + 16u * (uint32_t)l));
    R.b[0] = load16<true>(cp + ((uint32_t)(sb + 16 * nbc) + 16u * (uint32_t)l));
}

// The ring over a wave's items, as ring_loop (every step issues one item's
// loads, the padding at the front, the last N items drained without
// refills), with rotating parts.
// load(regs, rs, cursor) issues one item's loads (a cursor past the
// schedule reads the idle region).
template <int N, typename Regs, typename LoadF>
__device__ inline void rot_prologue(const RotSched& rs, Regs (&R)[N], LoadF&& load) {
    const int T = rs.total();
    const int pad = (T + N - 1) / N * N - T;
    RotCursor it;
    it.start(rs);
#pragma unroll
    for (int s = 0; s < N; ++s) {
        if (s < pad) {
            RotCursor none;
            none.j = rs.sc->tiles_wg;
            load(R[s], rs, none);
        } else {
            load(R[s], rs, it);
            it.next(rs);
        }
    }
}

template <int N, typename Regs, typename LoadF, typename ComputeF, typename KeepF>
__device__ inline void rot_loop(const RotSched& rs, Regs (&R)[N], LoadF&& load, ComputeF&& compute,
                                KeepF&& keep) {
    const Sched& sc = *rs.sc;
    const int T = rs.total();
    if (T == 0) return;
    const int P = (T + N - 1) / N * N, pad = P - T;
    RotCursor cur, nxt;
    cur.start(rs);
    nxt.start(rs);
    for (int q = pad; q < N; ++q) nxt.next(rs);  // the items the prologue requested
    float acc = 0.0f;
    auto consume = [&](Regs& r, int q) {
        if (q < pad) return;
        const int row = sc.row(cur.j);
        if (row < sc.n) {
            Sched s1 = sc;
            s1.part = cur.p;
            compute(r, s1, row, cur.m, acc);
        }
        if (cur.m == cur.ipt - 1) {
            keep(wave_sum(acc), cur.j, sc.group * sc.S + cur.p);
            acc = 0.0f;
        }
        cur.next(rs);
    };
    const int groups = P / N;
    for (int gi = 0; gi + 1 < groups; ++gi) {
#pragma unroll
        for (int s = 0; s < N; ++s) {
            consume(R[s], gi * N + s);
            load(R[s], rs, nxt);
            nxt.next(rs);
        }
    }
#pragma unroll
    for (int s = 0; s < N; ++s) consume(R[s], (groups - 1) * N + s);
}

// Split-K kernels that keep each tile's partial sums in LDS (res[tile]
// [group * S + part]) and add them once, after the row loop and one
// barrier, rather than meeting at two barriers per tile.
constexpr int kKeepTiles = 32;
template <int WAVES>
__host__ __device__ constexpr size_t lds_keep_bytes() {
    return (size_t)kKeepTiles * WAVES * sizeof(float);
}

// After the loop and a barrier: y[row] = the row's parts added in part
// order.
template <int WAVES>
__device__ inline void flush_parts(const Sched& sc, const float* res, float* y) {
    for (int i = (int)threadIdx.x; i < sc.tiles_wg * sc.groups; i += WAVES * kWave) {
        const int j = i / sc.groups, grp = i % sc.groups;
        const int row = ((int)blockIdx.x + j * sc.grid) * sc.groups + grp;
        if (row < sc.n) {
            const float* p = res + j * WAVES + grp * sc.S;
            float total = p[0];
            for (int q = 1; q < sc.S; ++q) total += p[q];
            y[row] = total;
        }
    }
}

// ------------------------------------------------------ activation staging
// Each path stages the activation in LDS in two steps: issue() puts this
// thread's first NR units in registers (before the weight prefetch, so
// waiting for them does not wait for the weights), commit() writes them and
// any remaining units to LDS.  The workgroup's thread count T is a template
// argument, not blockDim.x: on this target the block size is read from the
// dispatch's implicit arguments with a 16-bit vector load, and an address
// computed from it makes the wave wait for every load issued before it, so
// the weight prefetch would start one memory round trip late.

// Planar Q8_0 activation (q[k] then fp16 d[k/32]) -> LDS int4v q[C][2][64]
// (half h of block 64c+l) and float dx[C*64].
template <int NR, int T>
struct StageQ8 {
    int4v q[NR];
    uint16_t d[NR];
    __device__ void issue(const void* __restrict__ xin, int k, int C) {
        const int NB = k / kBlock;
        const int8_t* qx = static_cast<const int8_t*>(xin);
        const uint16_t* dx = reinterpret_cast<const uint16_t*>(qx + k);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = threadIdx.x + i * T;
            const int l = u % kWave, ch = u / kWave, h = ch & 1, c = ch >> 1;
            const int b = c * kWave + l;
            if (u < C * 2 * kWave && b < NB) q[i] = *reinterpret_cast<const int4v*>(qx + (int64_t)b * kBlock + 16 * h);
            const int bd = threadIdx.x + i * T;
            if (bd < NB) d[i] = dx[bd];
        }
    }
    __device__ void commit(const void* __restrict__ xin, int k, int C, int4v* lds_q, float* lds_dx) {
        const int NB = k / kBlock;
        const int8_t* qx = static_cast<const int8_t*>(xin);
        const uint16_t* dx = reinterpret_cast<const uint16_t*>(qx + k);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = threadIdx.x + i * T;
            const int l = u % kWave, c = (u / kWave) >> 1;
            if (u < C * 2 * kWave && c * kWave + l < NB) lds_q[u] = q[i];
            const int bd = threadIdx.x + i * T;
            if (bd < NB) lds_dx[bd] = half_bits_to_float(d[i]);
        }
        for (int u = threadIdx.x + NR * T; u < C * 2 * kWave; u += T) {
            const int l = u % kWave, ch = u / kWave, h = ch & 1, c = ch >> 1;
            const int b = c * kWave + l;
            if (b < NB) lds_q[u] = *reinterpret_cast<const int4v*>(qx + (int64_t)b * kBlock + 16 * h);
        }
        for (int b = threadIdx.x + NR * T; b < NB; b += T) lds_dx[b] = half_bits_to_float(dx[b]);
    }
};

// Requantized activation (the Q8_0 rule of quantize_act_q8_0) into the LDS
// layout of the int8 path: four lanes per 32-value block, eight values each
// (q8_quad_codes); every lane writes its eight codes (one 8-byte LDS store).
__device__ inline void requant_unit(const float4v v0, const float4v v1, int u, int4v* lds_q, float* lds_dx) {
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t lo, hi;
    const uint16_t d16 = q8_quad_codes(v, lo, hi);
    const int b = u >> 2, e = u & 3;
    const int c = b / kWave, l = b % kWave, h = e >> 1;
    uint32_t* dst = reinterpret_cast<uint32_t*>(lds_q + (c * 2 + h) * kWave + l) + 2 * (e & 1);
    dst[0] = lo;
    dst[1] = hi;
    if (e == 0) lds_dx[b] = half_bits_to_float(d16);
}

// f32 activation quantized with the Q8_0 rule into the same LDS layout (the
// codes and scales of quantize_act_q8_0): a unit is eight values, four
// units per 32-value block (requant_unit).  units = 4 x blocks and the
// workgroup is a whole number of waves, so the four lanes of a block are in
// the same wave and all (in)active together.
template <int NR, int T>
struct StageRequant {
    float4v v[NR][2];
    __device__ void issue(const void* __restrict__ xin, int k, int) {
        const int units = k / 8;
        const float4v* x4 = static_cast<const float4v*>(xin);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = threadIdx.x + i * T;
            if (u < units) {
                v[i][0] = x4[2 * u];
                v[i][1] = x4[2 * u + 1];
            }
        }
    }
    __device__ void commit(const void* __restrict__ xin, int k, int, int4v* lds_q, float* lds_dx) {
        const int units = k / 8;
        const float4v* x4 = static_cast<const float4v*>(xin);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = threadIdx.x + i * T;
            if (u < units) requant_unit(v[i][0], v[i][1], u, lds_q, lds_dx);
        }
        for (int u = threadIdx.x + NR * T; u < units; u += T)
            requant_unit(x4[2 * u], x4[2 * u + 1], u, lds_q, lds_dx);
    }
};

// LDS slot of the f32 staging layout of the dequantizing path for float4
// unit u (values 4u .. 4u+3): block b = u / 8 (= 64 c + l), group g = u % 8
// -> float4 (c * 8 + g) * 64 + l.
__device__ inline int f32_slot(int u) {
    const int b = u >> 3, g = u & 7, c = b / kWave, l = b % kWave;
    return (c * 8 + g) * kWave + l;
}

// ------------------------------------ residual + RMSNorm + requantization
// Arguments of residual_rmsnorm_q8_0 when a GEMV computes it in its
// prologue: h' = h + r (r nullable), y = h' / sqrt(mean h'^2 + eps) * g (g
// nullable), h' stored to h_out (nullable) by workgroup 0.
struct NormArgs {
    const float* h;
    const float* r;
    const float* g;
    float* h_out;
    float eps;
};

// Threads residual_rmsnorm_q8_0 runs for k values; thread t owns the units
// (eight values) t, t + T, t + 2T, ...
__host__ __device__ inline int norm_threads(int k) {
    const int units = k / 8;
    const int nt = (units + kWave - 1) / kWave * kWave;
    return nt > 1024 ? 1024 : (nt < kWave ? kWave : nt);
}

// The norm step as a GEMV's input staging, by a workgroup of T threads.  The
// mean of squares is reduced exactly as residual_rmsnorm_q8_0 reduces it:
// this workgroup plays that kernel's threads (thread vt = tid + m T),
// each summing its units in order with fused multiply-adds, then the same
// butterfly per wave and the wave partials in wave order; the values are
// then scaled and quantized with the same operations.  So the codes and
// scales in LDS are those that kernel writes, bit for bit.  With F32OUT the
// normalized values themselves are staged instead, in the f32 layout the
// dequantizing GEMV reads: they are that kernel's f32 output y, bit for
// bit.  Up to four
// units of the first pass are requested before the weight stream starts
// (issue); the rest, the reduction and the second pass come in commit.
// With one unit per norm thread (k <= 8192) both passes see the same units,
// so g is requested with them and the second pass reads nothing: one round
// trip to memory in all.
template <int T, bool F32OUT = false>
struct StageNorm {
    static_assert(T % kWave == 0 && 1024 % T == 0, "a whole number of waves dividing 1024 threads");
    static constexpr int MV = 1024 / T;  // most norm threads one thread plays
    NormArgs na;
    int k;
    float4v hv[4][2];
    float4v gv[4][2];  // g of the same units, when one unit per norm thread (k <= 8192)

    __device__ int pairs(int& nt, int& nu, int& units) const {
        units = k / 8;
        nt = norm_threads(k);
        nu = (units + nt - 1) / nt;
        return ((nt + T - 1) / T) * nu;
    }
    // loads h' of pairs p0 .. p0 + 3 (pair p: norm thread tid + (p / nu) T,
    // its (p % nu)-th unit)
    __device__ void load4(int p0, int P, int nt, int nu, int units) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int p = p0 + q, m = p / nu, i = p - m * nu;
            const int vt = (int)threadIdx.x + m * T, u = vt + i * nt;
            if (p < P && vt < nt && u < units) {
                const float4v* h4 = reinterpret_cast<const float4v*>(na.h) + 2 * u;
                hv[q][0] = h4[0];
                hv[q][1] = h4[1];
                if (na.r) {
                    const float4v* r4 = reinterpret_cast<const float4v*>(na.r) + 2 * u;
                    hv[q][0] += r4[0];
                    hv[q][1] += r4[1];
                }
            }
        }
    }
    __device__ void issue() {
        int nt, nu, units;
        const int P = pairs(nt, nu, units);
        load4(0, P, nt, nu, units);
        if (nu == 1 && na.g) {  // pair q is unit tid + q T: the second pass needs only g
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = (int)threadIdx.x + q * T;
                if (q < P && u < units) {
                    const float4v* g4 = reinterpret_cast<const float4v*>(na.g) + 2 * u;
                    gv[q][0] = g4[0];
                    gv[q][1] = g4[1];
                }
            }
        }
    }
    // scales h' of unit u by sc (and g), stores h' (workgroup 0) and
    // quantizes it into LDS
    __device__ void finish_unit(int u, float4v x0, float4v x1, bool has_g, float4v g0, float4v g1, float sc,
                                bool store_h, int4v* lds_q, float* lds_dx) const {
        if (store_h) {
            float4v* o4 = reinterpret_cast<float4v*>(na.h_out) + 2 * u;
            o4[0] = x0;
            o4[1] = x1;
        }
        const float a[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        float v[8];
        if (has_g) {
            const float gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (a[j] * sc) * gw[j];
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = a[j] * sc;
        }
        if constexpr (F32OUT) {
            float4v* lds_x = reinterpret_cast<float4v*>(lds_q);
            lds_x[f32_slot(2 * u)] = float4v{v[0], v[1], v[2], v[3]};
            lds_x[f32_slot(2 * u + 1)] = float4v{v[4], v[5], v[6], v[7]};
            (void)lds_dx;
        } else {
            requant_unit(float4v{v[0], v[1], v[2], v[3]}, float4v{v[4], v[5], v[6], v[7]}, u, lds_q, lds_dx);
        }
    }
    __device__ void commit(int4v* lds_q, float* lds_dx, float* scratch) {
        int nt, nu, units;
        const int P = pairs(nt, nu, units);
        float ss[MV];
#pragma unroll
        for (int mm = 0; mm < MV; ++mm) ss[mm] = 0.0f;
        for (int p0 = 0; p0 < P; p0 += 4) {
            if (p0 > 0) load4(p0, P, nt, nu, units);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p = p0 + q, m = p / nu, i = p - m * nu;
                const int vt = (int)threadIdx.x + m * T, u = vt + i * nt;
                if (p < P && vt < nt && u < units) {
                    const float a[8] = {hv[q][0].x, hv[q][0].y, hv[q][0].z, hv[q][0].w,
                                        hv[q][1].x, hv[q][1].y, hv[q][1].z, hv[q][1].w};
#pragma unroll
                    for (int mm = 0; mm < MV; ++mm) {
                        if (m == mm) {
#pragma unroll
                            for (int j = 0; j < 8; ++j) ss[mm] = __builtin_fmaf(a[j], a[j], ss[mm]);
                        }
                    }
                }
            }
        }
        const int lane = (int)threadIdx.x % kWave;
#pragma unroll
        for (int mm = 0; mm < MV; ++mm) {
            const float w = wave_sum(ss[mm]);
            const int vt = (int)threadIdx.x + mm * T;
            if (lane == 0 && vt < nt) scratch[vt / kWave] = w;
        }
        __syncthreads();
        float total = 0.0f;
        for (int w = 0; w < nt / kWave; ++w) total += scratch[w];
        const float sc = 1.0f / __builtin_sqrtf(total / (float)k + na.eps);
        const bool store_h = na.h_out != nullptr && blockIdx.x == 0;
        if (nu == 1) {
            // one unit per norm thread: pair q of the first pass is unit
            // tid + q T, still in registers with its g
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int u = (int)threadIdx.x + q * T;
                if (q < P && u < units)
                    finish_unit(u, hv[q][0], hv[q][1], na.g != nullptr, gv[q][0], gv[q][1], sc, store_h, lds_q,
                                lds_dx);
            }
        } else {
            second_pass(units, sc, store_h, lds_q, lds_dx);
        }
        // only workgroup 0 stores h': wait for every memory operation here,
        // so that the row loop starts from the same count on every path and
        // its waits stay exact (s_waitcnt vmcnt(0), no other counter)
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    __device__ void second_pass(int units, float sc, bool store_h, int4v* lds_q, float* lds_dx) const {
        for (int u = (int)threadIdx.x; u < units; u += T) {
            const float4v* h4 = reinterpret_cast<const float4v*>(na.h) + 2 * u;
            float4v x0 = h4[0], x1 = h4[1];
            if (na.r) {
                const float4v* r4 = reinterpret_cast<const float4v*>(na.r) + 2 * u;
                x0 += r4[0];
                x1 += r4[1];
            }
            float4v g0 = {}, g1 = {};
            if (na.g) {
                const float4v* g4 = reinterpret_cast<const float4v*>(na.g) + 2 * u;
                g0 = g4[0];
                g1 = g4[1];
            }
            finish_unit(u, x0, x1, na.g != nullptr, g0, g1, sc, store_h, lds_q, lds_dx);
        }
    }
};

// f32 activation for the dequantizing path: float4 v (values 4v..4v+3, block
// b = v/8, group g = v%8) -> LDS float4v x[C][8][64] at (c*8+g)*64 + l.
template <int NR, int T>
struct StageF32 {
    float4v v[NR];
    __device__ static int slot(int u) { return f32_slot(u); }
    __device__ void issue(const float* __restrict__ x, int k) {
        const float4v* x4 = reinterpret_cast<const float4v*>(x);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = threadIdx.x + i * T;
            if (u < k / 4) v[i] = x4[u];
        }
    }
    __device__ void commit(const float* __restrict__ x, int k, float4v* lds_x) {
        const float4v* x4 = reinterpret_cast<const float4v*>(x);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = threadIdx.x + i * T;
            if (u < k / 4) lds_x[slot(u)] = v[i];
        }
        for (int u = threadIdx.x + NR * T; u < k / 4; u += T) lds_x[slot(u)] = x4[u];
    }
};

// f32 activation for the bf16 path: element e = 1024c + 512h + 8l + 4j ->
// LDS float4v x[C'][2][2][64] at ((c*2+h)*2+j)*64 + l.
template <int NR, int T>
struct StageBf16x {
    float4v v[NR];
    __device__ static int slot(int u) {
        const int e = 4 * u;
        const int c = e >> 10, h = (e >> 9) & 1, l = (e >> 3) & 63, j = (e >> 2) & 1;
        return ((c * 2 + h) * 2 + j) * kWave + l;
    }
    __device__ void issue(const float* __restrict__ x, int k) {
        const float4v* x4 = reinterpret_cast<const float4v*>(x);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = threadIdx.x + i * T;
            if (u < k / 4) v[i] = x4[u];
        }
    }
    __device__ void commit(const float* __restrict__ x, int k, float4v* lds_x) {
        const float4v* x4 = reinterpret_cast<const float4v*>(x);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = threadIdx.x + i * T;
            if (u < k / 4) lds_x[slot(u)] = v[i];
        }
        for (int u = threadIdx.x + NR * T; u < k / 4; u += T) lds_x[slot(u)] = x4[u];
    }
};

// ------------------------------------------------------ Q8_0 x f32 (deq)
__device__ inline float dot4_i8_f32(int w, float4v x, float acc) {
    acc = __builtin_fmaf((float)(int8_t)(w & 0xFF), x.x, acc);
    acc = __builtin_fmaf((float)(int8_t)((w >> 8) & 0xFF), x.y, acc);
    acc = __builtin_fmaf((float)(int8_t)((w >> 16) & 0xFF), x.z, acc);
    acc = __builtin_fmaf((float)(int8_t)(w >> 24), x.w, acc);
    return acc;
}

// ---------------------------------------------------------- BF16 x f32
__device__ inline float dot_bf16x8(int4v w, float4v x0, float4v x1, float acc) {
    acc = __builtin_fmaf(__uint_as_float((uint32_t)w.x << 16), x0.x, acc);
    acc = __builtin_fmaf(__uint_as_float((uint32_t)w.x & 0xFFFF0000u), x0.y, acc);
    acc = __builtin_fmaf(__uint_as_float((uint32_t)w.y << 16), x0.z, acc);
    acc = __builtin_fmaf(__uint_as_float((uint32_t)w.y & 0xFFFF0000u), x0.w, acc);
    acc = __builtin_fmaf(__uint_as_float((uint32_t)w.z << 16), x1.x, acc);
    acc = __builtin_fmaf(__uint_as_float((uint32_t)w.z & 0xFFFF0000u), x1.y, acc);
    acc = __builtin_fmaf(__uint_as_float((uint32_t)w.w << 16), x1.z, acc);
    acc = __builtin_fmaf(__uint_as_float((uint32_t)w.w & 0xFFFF0000u), x1.w, acc);
    return acc;
}

template <int U>
struct Bf16Regs {
    int4v a[U], b[U];
};

// Requests item `it`: U 1024-element chunks of one bf16 row, 2U loads
// whether or not the item, the row or a chunk exists (those read the idle
// region).  Lanes past the end of a ragged row re-read its last 8 elements
// (not divergent); compute skips them.
template <int U>
__device__ inline void bf16_load_item(Bf16Regs<U>& r, gptr<uint16_t> W, int k, const Sched& sc,
                                      const ItemCursor& it) {
    const int lane = threadIdx.x % kWave;
    const int row = it.j < sc.tiles_wg ? sc.row(it.j) : sc.n;
    const bool has_row = row < sc.n;
    const gptr<uint8_t> rowp = (gptr<uint8_t>)(W + (int64_t)(has_row ? row : 0) * k);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = sc.chunk(it.m, u);
        const bool real = has_row && c < sc.C;
        const int e0 = c * 1024 + 8 * lane;
        const int ea = e0 < k ? e0 : k - 8;
        const int eb = e0 + 512 < k ? e0 + 512 : k - 8;
        // a wave-uniform base (the row or the idle region) plus a 32-bit
        // per-lane byte offset: a scalar base register in each load
        const gptr<uint8_t> base = real ? rowp : idle_bytes();
        r.a[u] = load16<true>(base + (real ? 2u * (uint32_t)ea : 16u * (uint32_t)lane));
        r.b[u] = load16<true>(base + (real ? 2u * (uint32_t)eb : 16u * (uint32_t)lane));
    }
}

// Makes a loaded value opaque to the optimizer at its point of use, so that
// byte or half extraction is not folded back into the (conditional) block
// that issued the load -- there it would force an immediate wait for the
// load and defeat the pipelining.
__device__ inline void opaque(int4v& v) { asm volatile("" : "+v"(v)); }

// ------------------------------------------------------- item compute
// One item of the int8 path: U chunks, one 32-weight block per lane each;
// s = exact int32 block dot (8 x v_dot4), acc += (d_w * d_x) * s.
template <int U, bool DEBUG>
__device__ inline void q8_i8_item(const Q8Regs<U>& r, const Sched& sc, int m, int NB, const int4v* lds_q,
                                  const float* lds_dx, int row, int32_t* dots, float& acc) {
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = sc.chunk(m, u);
        const int blk = c * kWave + lane;
        if (c < sc.C && blk < NB) {
            const int4v xa = lds_q[(c * 2 + 0) * kWave + lane];
            const int4v xb = lds_q[(c * 2 + 1) * kWave + lane];
            int s = 0;
            s = __builtin_amdgcn_sdot4(r.a[u].x, xa.x, s, false);
            s = __builtin_amdgcn_sdot4(r.a[u].y, xa.y, s, false);
            s = __builtin_amdgcn_sdot4(r.a[u].z, xa.z, s, false);
            s = __builtin_amdgcn_sdot4(r.a[u].w, xa.w, s, false);
            s = __builtin_amdgcn_sdot4(r.b[u].x, xb.x, s, false);
            s = __builtin_amdgcn_sdot4(r.b[u].y, xb.y, s, false);
            s = __builtin_amdgcn_sdot4(r.b[u].z, xb.z, s, false);
            s = __builtin_amdgcn_sdot4(r.b[u].w, xb.w, s, false);
            if constexpr (DEBUG) dots[(int64_t)row * NB + blk] = s;
            const float t = half_bits_to_float(r.sc[u]) * lds_dx[blk];
            acc = __builtin_fmaf(t, (float)s, acc);
        }
    }
    (void)row;
    (void)dots;
}

// One item of the dequantizing path: acc += d_w * sum_i q_i x_i per block.
template <int U>
__device__ inline void q8_f32_item(const Q8Regs<U>& r, const Sched& sc, int m, int NB, const float4v* lds_x,
                                   float& acc) {
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = sc.chunk(m, u);
        if (c < sc.C && c * kWave + lane < NB) {
            const float4v* xv = lds_x + (size_t)c * 8 * kWave + lane;
            int4v wa = r.a[u], wb = r.b[u];
            opaque(wa);
            opaque(wb);
            float bs = 0.0f;
            bs = dot4_i8_f32(wa.x, xv[0 * kWave], bs);
            bs = dot4_i8_f32(wa.y, xv[1 * kWave], bs);
            bs = dot4_i8_f32(wa.z, xv[2 * kWave], bs);
            bs = dot4_i8_f32(wa.w, xv[3 * kWave], bs);
            bs = dot4_i8_f32(wb.x, xv[4 * kWave], bs);
            bs = dot4_i8_f32(wb.y, xv[5 * kWave], bs);
            bs = dot4_i8_f32(wb.z, xv[6 * kWave], bs);
            bs = dot4_i8_f32(wb.w, xv[7 * kWave], bs);
            acc = __builtin_fmaf(half_bits_to_float(r.sc[u]), bs, acc);
        }
    }
}

}  // namespace
}  // namespace wsg
