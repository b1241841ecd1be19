// Batch-1 decode GEMV kernels for gfx950: y = W.x streaming a whole weight
// matrix against one activation vector (emit_qwen38_generate, "Where the
// speed comes from"; qwen3-8b-rtx4080-cutedsl, "Decode GEMV path"; GPU
// Kernel Lab, "What we built": split-K, warp-reduced decode GEMV).
//
// Mapping (all paths):
//  * A persistent grid of workgroups of WAVES wave64s.  Each workgroup first
//    stages the whole activation in LDS, in the order the lanes consume it,
//    then walks row tiles t = blockIdx.x, blockIdx.x + gridDim.x, ...
//  * A tile holds WAVES/S rows; S waves share one row and split its chunks
//    (split-K inside the workgroup: chunk c goes to wave-part c % S).  Each
//    wave reduces over its 64 lanes with a fixed butterfly, the S partials
//    meet in LDS and are added in part order, so a row's result does not
//    depend on where or when it was computed.  No atomics, no cross-workgroup
//    reduction.
//  * Lane l of a wave owns block l of every 64-block chunk of a row: with the
//    device layout it gets the block's 32 codes from two contiguous 1 KB
//    wave loads (16 bytes per lane) and its scale from one 128-byte load.
//  * Each wave keeps a ring of weight items (U chunks each: three one-chunk
//    items by default) in registers: while one item is consumed the others
//    are in flight.  Every step of the row loop issues the same loads
//    (absent items read a small idle region), so the compiler waits for one
//    ring set at a time rather than for every outstanding load.
//  * No MFMA: at batch 1 there is one multiply-add per weight and no reuse.
#include "common.hpp"
#include "gemv_device.hpp"
#include "internal.hpp"
#include "timeline.hpp"

#include <atomic>
#include <cstdlib>
#include <type_traits>
#include <map>
#include <tuple>
#include <mutex>
#include <utility>

namespace wsg {
namespace {

// Register sets in each wave's ring of weight items of U chunks (one
// consumed while the others are in flight): three one-chunk items, or two
// items of two or more chunks.
// (Measured on the 27B and 8B shapes: four one-chunk items for unsplit
// rows, or five for split ones, stream 2-10% slower -- more requests in
// flight only lengthen the queues; six spill.)
constexpr int kRing1 = 3, kRingSplit = 3;
template <int U, int S = 1>
constexpr int kRingSets = U == 1 ? (S > 1 ? kRingSplit : kRing1) : 2;

// ------------------------------------------------ Q8_0 x int8 (and requant)
// The int8 path's body; `stage` fills the activation's LDS layout:
// stage.issue() requests the input before the first weight items are
// requested, stage.commit(lds_q, lds_dx, scratch) completes it (scratch:
// LDS the row loop has not started to use).
template <int WAVES, int S, int U, bool DEBUG, bool ARGMAX, typename Stage>
__device__ __attribute__((always_inline)) inline void q8_i8_body(const uint8_t* __restrict__ W, int n, int k,
                                                                 float* __restrict__ y, int32_t* __restrict__ dots,
                                                                 uint64_t* __restrict__ keys, Stage& stage) {
    static_assert(WAVES % S == 0, "S must divide WAVES");
    extern __shared__ __align__(16) uint8_t smem[];
    const int C = (int)chunk_count(k);
    const int NB = k / kBlock;
    const int nl = NB - (C - 1) * kChunkBlocks;
    const int sbl = (int)scale_section_bytes(nl);
    const int64_t row_bytes = packed_row_bytes(k);
    int4v* lds_q = reinterpret_cast<int4v*>(smem);
    float* lds_dx = reinterpret_cast<float*>(smem + (size_t)C * 2 * kWave * 16);
    float* lds_part = reinterpret_cast<float*>(smem + lds_q8act_bytes(C));
    uint64_t* lds_key = reinterpret_cast<uint64_t*>(smem + ((lds_q8act_bytes(C) + WAVES * 4 + 15) & ~size_t(15)));
    const int lane = threadIdx.x % kWave;

    WSG_TL_BEGIN();
    const Sched sc(C, S, U, WAVES, n, (n + WAVES / S - 1) / (WAVES / S));
    const gptr<uint8_t> Wg = (gptr<uint8_t>)W;
    auto load = [&](Q8Regs<U>& r, const ItemCursor& it) { q8_load_item<U>(r, Wg, row_bytes, sc, nl, sbl, it); };
    auto compute = [&](const Q8Regs<U>& r, int row, int m, float& acc) {
        q8_i8_item<U, DEBUG>(r, sc, m, NB, lds_q, lds_dx, row, dots, acc);
    };

    // split rows with one-chunk items: rotating parts, partials kept in LDS
    // (rot_loop, flush_parts) while the workgroup's tiles fit
    constexpr bool kRot = S > 1 && U == 1 && !DEBUG && !ARGMAX;
    const int wave = wave_id();
    const bool rot = kRot && sc.tiles_wg <= kKeepTiles;
    float* lds_res = reinterpret_cast<float*>(smem + lds_q8act_bytes(C) + lds_tail_bytes<WAVES>());
    RotSched rs;
    rs.set(sc, wave);
    auto rload = [&](Q8Regs<1>& r, const RotSched& rs_, const RotCursor& it) {
        q8_load_rot(r, Wg, row_bytes, nl, sbl, rs_, it);
    };
    auto prologue = [&](Q8Regs<U> (&R_)[kRingSets<U, S>]) {
        if constexpr (kRot) {
            if (rot) {
                rot_prologue(rs, R_, rload);
                return;
            }
        }
        ring_prologue(sc, R_, load);
    };

    Q8Regs<U> R[kRingSets<U, S>];
    stage.issue();
    __builtin_amdgcn_sched_barrier(0);
    prologue(R);
    __builtin_amdgcn_sched_barrier(0);
    stage.commit(lds_q, lds_dx, lds_res);
    __syncthreads();
    WSG_TL_STAGED();
    if constexpr (kRot) {
        if (rot) {
            if (threadIdx.x % kWave < (unsigned)sc.tiles_wg) {
                const int t = (int)(threadIdx.x % kWave);
                if (rs.items(t) == 0) lds_res[t * WAVES + sc.group * S + rs.part(t)] = 0.0f;
            }
            rot_loop(rs, R, rload,
                     [&](const Q8Regs<1>& r, const Sched& s1, int row, int m, float& acc) {
                         q8_i8_item<1, false>(r, s1, m, NB, lds_q, lds_dx, row, nullptr, acc);
                     },
                     [&](float acc, int t, int slot) {
                         if (lane == 0) lds_res[t * WAVES + slot] = acc;
                     });
            WSG_TL_LOOP_END();
            __syncthreads();
            flush_parts<WAVES>(sc, lds_res, y);
            WSG_TL_END(y);
            return;
        }
    }
    uint64_t best = 0;
    ring_loop(sc, R, load, compute, [&](float acc, int, int row, bool) {
        finish_row<WAVES, S, ARGMAX>(acc, row, n, lane, wave, lds_part, y, best);
    });
    WSG_TL_LOOP_END();
    if constexpr (ARGMAX) write_block_key<WAVES>(best, lane, wave, lds_key, keys);
    WSG_TL_END(y);
}

// Staging of the int8 path's input: a quantize_act_q8_0 output, or f32
// requantized in the workgroup.
template <int ACT, int T>
struct StageInput {
    const void* xin;
    int k, C;
    typename std::conditional<ACT == kActRequant, StageRequant<4, T>, StageQ8<4, T>>::type st;
    __device__ void issue() { st.issue(xin, k, C); }
    __device__ void commit(int4v* lds_q, float* lds_dx, float*) { st.commit(xin, k, C, lds_q, lds_dx); }
};

// f32 input of the dequantizing path (the SwiGLU kernel's W8A16 form).
template <int T>
struct StageInput<kActF32, T> {
    const void* xin;
    int k, C;
    StageF32<4, T> st;
    __device__ void issue() { st.issue(static_cast<const float*>(xin), k); }
    __device__ void commit(int4v* lds, float*, float*) {
        st.commit(static_cast<const float*>(xin), k, reinterpret_cast<float4v*>(lds));
    }
};

template <int WAVES, int S, int U, int ACT, bool NT, bool DEBUG, bool ARGMAX>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(4)))
q8_i8_kernel(const uint8_t* __restrict__ W, int n, int k, const void* __restrict__ xin, float* __restrict__ y,
             int32_t* __restrict__ dots, uint64_t* __restrict__ keys) {
    static_assert(NT, "the weight stream is always loaded non-temporally");
    StageInput<ACT, WAVES * kWave> stage{xin, k, (int)chunk_count(k), {}};
    q8_i8_body<WAVES, S, U, DEBUG, ARGMAX>(W, n, k, y, dots, keys, stage);
}

// The gate+up GEMV with the SwiGLU epilogue (GPU Kernel Lab, "What we
// built", "Decode integration": the dual gate/up projection fused with
// SwiGLU at batch 1): W holds 2 n_ff rows, gate rows first, and
// y[p] = silu(g_p) u_p with g_p = row p . x and u_p = row n_ff + p . x.
// Each wave takes one output p per tile and walks the 2C chunks of both
// rows as one sequence (gate chunks, then up chunks), with one accumulator
// per row, so each half is reduced exactly as the unsplit kernel reduces
// that row (per-lane fused multiply-adds in chunk order, then the
// butterfly) and only the n_ff products are stored.  With f32 activations
// (ACT = kActF32, the W8A16 form of the same page's "Quantization
// experiments") each block is dequantized against the f32 input as in the
// dequantizing GEMV, so each half equals that GEMV's row bit for bit.
template <int WAVES, int ACT>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(4)))
q8_i8_swiglu_kernel(const uint8_t* __restrict__ W, int n_ff, int k, const void* __restrict__ xin,
                    float* __restrict__ y) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int C = (int)chunk_count(k);
    const int NB = k / kBlock;
    const int nl = NB - (C - 1) * kChunkBlocks;
    const int sbl = (int)scale_section_bytes(nl);
    const int64_t row_bytes = packed_row_bytes(k);
    constexpr bool F32 = ACT == kActF32;
    int4v* lds_q = reinterpret_cast<int4v*>(smem);
    float* lds_dx = reinterpret_cast<float*>(smem + (size_t)C * 2 * kWave * 16);
    const float4v* lds_x = reinterpret_cast<const float4v*>(smem);
    const size_t act_bytes = F32 ? lds_f32act_bytes(C) : lds_q8act_bytes(C);
    float* lds_res = reinterpret_cast<float*>(smem + act_bytes + lds_tail_bytes<WAVES>());
    const int lane = threadIdx.x % kWave;
    const Sched sc(2 * C, 1, 1, WAVES, n_ff, (n_ff + WAVES - 1) / WAVES);
    const gptr<uint8_t> Wg = (gptr<uint8_t>)W;
    // item m of output p: chunk m of gate row p (m < C) or chunk m - C of up
    // row n_ff + p; past the schedule the idle region (see q8_load_item)
    auto load = [&](Q8Regs<1>& r, const ItemCursor& it) {
        const int p = it.j < sc.tiles_wg ? sc.row(it.j) : sc.n;
        const int m = sc.chunk(it.m, 0);
        const bool up = m >= C;
        const int c = up ? m - C : m;
        const bool real = p < sc.n && m < 2 * C;
        const bool last = c == C - 1;
        const int nbc = last ? nl : kChunkBlocks;
        const int sb = last ? sbl : 2 * kChunkBlocks;
        const int l = lane < nbc ? lane : nbc - 1;
        const int64_t row = real ? (int64_t)p + (up ? n_ff : 0) : 0;
        const gptr<uint8_t> cp = real ? Wg + row * row_bytes + (int64_t)c * kFullChunkBytes : idle_bytes();
        r.sc[0] = load_u16<true>(cp + 2u * (uint32_t)l);
        r.a[0] = load16<true>(cp + ((uint32_t)sb + 16u * (uint32_t)l));
        r.b[0] = load16<true>(cp + ((uint32_t)(sb + 16 * nbc) + 16u * (uint32_t)l));
    };
    float acc_up = 0.0f;
    // one block per lane, as q8_i8_item: exact int32 dot, then (d_w d_x) s
    auto compute = [&](const Q8Regs<1>& r, int, int m, float& acc_gate) {
        const bool up = m >= C;
        const int c = up ? m - C : m;
        const int blk = c * kWave + lane;
        if (blk < NB) {
            float& acc = up ? acc_up : acc_gate;
            if constexpr (F32) {
                // as q8_f32_item: d_w times the block's f32 dot
                const float4v* xv = lds_x + (size_t)c * 8 * kWave + lane;
                int4v wa = r.a[0], wb = r.b[0];
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
                acc = __builtin_fmaf(half_bits_to_float(r.sc[0]), bs, acc);
            } else {
                const int4v xa = lds_q[(c * 2 + 0) * kWave + lane];
                const int4v xb = lds_q[(c * 2 + 1) * kWave + lane];
                int d = 0;
                d = __builtin_amdgcn_sdot4(r.a[0].x, xa.x, d, false);
                d = __builtin_amdgcn_sdot4(r.a[0].y, xa.y, d, false);
                d = __builtin_amdgcn_sdot4(r.a[0].z, xa.z, d, false);
                d = __builtin_amdgcn_sdot4(r.a[0].w, xa.w, d, false);
                d = __builtin_amdgcn_sdot4(r.b[0].x, xb.x, d, false);
                d = __builtin_amdgcn_sdot4(r.b[0].y, xb.y, d, false);
                d = __builtin_amdgcn_sdot4(r.b[0].z, xb.z, d, false);
                d = __builtin_amdgcn_sdot4(r.b[0].w, xb.w, d, false);
                const float t = half_bits_to_float(r.sc[0]) * lds_dx[blk];
                acc = __builtin_fmaf(t, (float)d, acc);
            }
        }
    };
    Q8Regs<1> R[kRingSets<1, 1>];
    StageInput<ACT, WAVES * kWave> stage{xin, k, C, {}};
    stage.issue();
    __builtin_amdgcn_sched_barrier(0);
    ring_prologue(sc, R, load);
    __builtin_amdgcn_sched_barrier(0);
    stage.commit(lds_q, lds_dx, lds_res);
    __syncthreads();
    ring_loop(sc, R, load, compute, [&](float gate, int, int p, bool valid) {
        const float upv = wave_sum(acc_up);
        acc_up = 0.0f;
        // silu(g) u; exp(-g) overflowing to +inf for very negative g gives -0
        if (valid && lane == 0) y[p] = gate / (1.0f + expf(-gate)) * upv;
    });
}

// ------------------------------------------------ 4-bit weights x int8
// The W4 GEMV (qwen3-8b-rtx4080-cutedsl, "W4A16 dequant-fused GEMM": the
// weights stream at 4 bits; GPU Kernel Lab, "Quantization experiments"):
// the int8 path's schedule, staging and ring with a 4-bit item: per lane
// one 16-byte load (its block's 32 codes) and the block's scale.  The
// stored codes are n = q + 8 in [1, 15], so with sdot4 over the unpacked
// nibbles s = sum n x - 8 sum x = sum q x, exact in int32; then
// acc += (d_w d_x) s as in the int8 path.  8 sum x depends on the
// activation block only: each workgroup computes it once per block into
// LDS after the staging, which halves the dot work per item.
struct Q4Regs {
    int4v a;
    uint16_t sc;
};

constexpr int kRingQ4 = 3;

// sum_i q_w,i q_x,i of block c * 64 + lane: the nibbles n = q_w + 8 dotted
// with the staged int8 codes, less the block's 8 sum x from LDS (exact).
__device__ inline int q4_block_dot(const Q4Regs& r, int c, int lane, const int4v* lds_q, const int* lds_sx8) {
    const int4v xa = lds_q[(c * 2 + 0) * kWave + lane];
    const int4v xb = lds_q[(c * 2 + 1) * kWave + lane];
    int4v wa = r.a;
    opaque(wa);
    const uint32_t w4[4] = {(uint32_t)wa.x, (uint32_t)wa.y, (uint32_t)wa.z, (uint32_t)wa.w};
    const int x4a[4] = {xa.x, xa.y, xa.z, xa.w}, x4b[4] = {xb.x, xb.y, xb.z, xb.w};
    int dn = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        dn = __builtin_amdgcn_sdot4((int)(w4[q] & 0x0F0F0F0Fu), x4a[q], dn, false);
        dn = __builtin_amdgcn_sdot4((int)((w4[q] >> 4) & 0x0F0F0F0Fu), x4b[q], dn, false);
    }
    return dn - lds_sx8[c * kWave + lane];
}

// 8 sum x of every staged block (block c * 64 + l: words (2c) * 64 + l and
// (2c + 1) * 64 + l of lds_q), by the T threads of the workgroup.
template <int T>
__device__ inline void q4_block_sums(const int4v* lds_q, int* lds_sx8, int C) {
    for (int b = threadIdx.x; b < C * kWave; b += T) {
        const int4v xa = lds_q[(b / kWave * 2) * kWave + b % kWave];
        const int4v xb = lds_q[(b / kWave * 2 + 1) * kWave + b % kWave];
        int sx = 0;
        sx = __builtin_amdgcn_sdot4(0x01010101, xa.x, sx, false);
        sx = __builtin_amdgcn_sdot4(0x01010101, xa.y, sx, false);
        sx = __builtin_amdgcn_sdot4(0x01010101, xa.z, sx, false);
        sx = __builtin_amdgcn_sdot4(0x01010101, xa.w, sx, false);
        sx = __builtin_amdgcn_sdot4(0x01010101, xb.x, sx, false);
        sx = __builtin_amdgcn_sdot4(0x01010101, xb.y, sx, false);
        sx = __builtin_amdgcn_sdot4(0x01010101, xb.z, sx, false);
        sx = __builtin_amdgcn_sdot4(0x01010101, xb.w, sx, false);
        lds_sx8[b] = 8 * sx;
    }
}

// `stage` fills the activation's LDS layout as in q8_i8_body: a staged
// int8 input (StageInput) or the residual add + RMSNorm + re-quantization
// (StageNorm).
template <int WAVES, int S, typename Stage>
__device__ __attribute__((always_inline)) inline void q4_i8_body(const uint8_t* __restrict__ W, int n, int k,
                                                                 float* __restrict__ y, Stage& stage) {
    static_assert(WAVES % S == 0, "S must divide WAVES");
    extern __shared__ __align__(16) uint8_t smem[];
    const int C = (int)chunk_count(k);
    const int NB = k / kBlock;
    const int nl = NB - (C - 1) * kChunkBlocks;
    const int sbl = (int)scale_section_bytes(nl);
    const int64_t row_bytes = q4_row_bytes(k);
    int4v* lds_q = reinterpret_cast<int4v*>(smem);
    float* lds_dx = reinterpret_cast<float*>(smem + (size_t)C * 2 * kWave * 16);
    float* lds_res = reinterpret_cast<float*>(smem + lds_q8act_bytes(C) + lds_tail_bytes<WAVES>());
    int* lds_sx8 = reinterpret_cast<int*>(smem + lds_q8act_bytes(C) + lds_tail_bytes<WAVES>() +
                                          lds_keep_bytes<WAVES>());
    float* lds_part = reinterpret_cast<float*>(smem + lds_q8act_bytes(C));
    const int lane = threadIdx.x % kWave;
    const int wave = wave_id();
    const Sched sc(C, S, 1, WAVES, n, (n + WAVES / S - 1) / (WAVES / S));
    const gptr<uint8_t> Wg = (gptr<uint8_t>)W;
    // chunk c of a row (row n or chunk C: the idle region)
    auto load_rc = [&](Q4Regs& r, int row, int c) {
        const bool real = row < sc.n && c < C;
        const bool last = c == C - 1;
        const int nbc = last ? nl : kChunkBlocks;
        const int sb = last ? sbl : 2 * kChunkBlocks;
        const int l = lane < nbc ? lane : nbc - 1;
        const gptr<uint8_t> cp = real ? Wg + (int64_t)row * row_bytes + (int64_t)c * kFullChunkBytesQ4 : idle_bytes();
        r.sc = load_u16<true>(cp + 2u * (uint32_t)l);
        r.a = load16<true>(cp + ((uint32_t)sb + 16u * (uint32_t)l));
    };
    auto compute_c = [&](const Q4Regs& r, int c, float& acc) {
        const int blk = c * kWave + lane;
        if (blk < NB) {
            const int s = q4_block_dot(r, c, lane, lds_q, lds_sx8);
            const float t = half_bits_to_float(r.sc) * lds_dx[blk];
            acc = __builtin_fmaf(t, (float)s, acc);
        }
    };
    // chunk m of the wave's row and part; past the schedule the idle region
    auto load = [&](Q4Regs& r, const ItemCursor& it) {
        load_rc(r, it.j < sc.tiles_wg ? sc.row(it.j) : sc.n, sc.chunk(it.m, 0));
    };
    auto compute = [&](const Q4Regs& r, int, int m, float& acc) { compute_c(r, sc.chunk(m, 0), acc); };
    // split rows: rotating parts with the partials kept in LDS while the
    // workgroup's tiles fit, as in the int8 path (rot_loop, flush_parts)
    constexpr bool kRot = S > 1;
    const bool rot = kRot && sc.tiles_wg <= kKeepTiles;
    RotSched rs;
    rs.set(sc, wave);
    auto rload = [&](Q4Regs& r, const RotSched& rs_, const RotCursor& it) {
        const bool has_item = it.j < rs_.sc->tiles_wg;
        load_rc(r, has_item ? sc.row(it.j) : sc.n, has_item ? it.p + S * it.m : C);
    };
    Q4Regs R[kRingQ4];
    stage.issue();
    __builtin_amdgcn_sched_barrier(0);
    if (rot)
        rot_prologue(rs, R, rload);
    else
        ring_prologue(sc, R, load);
    __builtin_amdgcn_sched_barrier(0);
    stage.commit(lds_q, lds_dx, lds_res);
    __syncthreads();
    q4_block_sums<WAVES * kWave>(lds_q, lds_sx8, C);
    __syncthreads();
    if constexpr (kRot) {
        if (rot) {
            if (threadIdx.x % kWave < (unsigned)sc.tiles_wg) {
                const int t = (int)(threadIdx.x % kWave);
                if (rs.items(t) == 0) lds_res[t * WAVES + sc.group * S + rs.part(t)] = 0.0f;
            }
            rot_loop(rs, R, rload,
                     [&](const Q4Regs& r, const Sched& s1, int, int m, float& acc) {
                         compute_c(r, s1.chunk(m, 0), acc);
                     },
                     [&](float acc, int t, int slot) {
                         if (lane == 0) lds_res[t * WAVES + slot] = acc;
                     });
            __syncthreads();
            flush_parts<WAVES>(sc, lds_res, y);
            return;
        }
    }
    uint64_t best = 0;
    ring_loop(sc, R, load, compute, [&](float acc, int, int row, bool) {
        finish_row<WAVES, S, false>(acc, row, n, lane, wave, lds_part, y, best);
    });
}

template <int WAVES, int S, int ACT>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(4)))
q4_i8_kernel(const uint8_t* __restrict__ W, int n, int k, const void* __restrict__ xin, float* __restrict__ y) {
    StageInput<ACT, WAVES * kWave> stage{xin, k, (int)chunk_count(k), {}};
    q4_i8_body<WAVES, S>(W, n, k, y, stage);
}

// The W4 GEMV fed by the residual add + RMSNorm + re-quantization of
// residual_rmsnorm_q8_0, computed by every workgroup in its prologue, as
// q8_i8_norm_kernel does for Q8_0 weights: the same codes and scales, bit
// for bit.
template <int WAVES, int S>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(4)))
q4_i8_norm_kernel(const uint8_t* __restrict__ W, int n, int k, NormArgs na, float* __restrict__ y) {
    StageNorm<WAVES * kWave> stage{na, k, {}};
    q4_i8_body<WAVES, S>(W, n, k, y, stage);
}

// The 4-bit gate+up GEMV with the SwiGLU epilogue, two waves per output:
// the waves of a workgroup pair up (2g, 2g + 1) and each pair takes one
// output p per tile, the even wave gate row p and the odd wave up row
// n_ff + p, each walking all C chunks of its row as the plain W4 kernel
// walks a row (so each half is reduced exactly as that kernel reduces the
// row).  Every wave streams one row at a time, as in the plain kernel,
// instead of one wave walking both rows of an output.  The halves wait in
// LDS (up to kKeepTiles tiles per workgroup) and meet after the row loop,
// so the stream has no workgroup barrier; with more tiles the pair meets
// at the end of each tile.
template <int WAVES, int ACT>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(4)))
q4_i8_swiglu_kernel(const uint8_t* __restrict__ W, int n_ff, int k, const void* __restrict__ xin,
                    float* __restrict__ y) {
    static_assert(WAVES % 2 == 0, "waves pair up");
    extern __shared__ __align__(16) uint8_t smem[];
    const int C = (int)chunk_count(k);
    const int NB = k / kBlock;
    const int nl = NB - (C - 1) * kChunkBlocks;
    const int sbl = (int)scale_section_bytes(nl);
    const int64_t row_bytes = q4_row_bytes(k);
    int4v* lds_q = reinterpret_cast<int4v*>(smem);
    float* lds_dx = reinterpret_cast<float*>(smem + (size_t)C * 2 * kWave * 16);
    float* lds_part = reinterpret_cast<float*>(smem + lds_q8act_bytes(C));
    float* lds_res = reinterpret_cast<float*>(smem + lds_q8act_bytes(C) + lds_tail_bytes<WAVES>());
    int* lds_sx8 = reinterpret_cast<int*>(smem + lds_q8act_bytes(C) + lds_tail_bytes<WAVES>() +
                                          lds_keep_bytes<WAVES>());
    const int lane = threadIdx.x % kWave;
    const int wave = wave_id();
    // a schedule of 2C chunks in two parts has C items per wave and part =
    // wave % 2; item m of either part is chunk m of that part's row
    const Sched sc(2 * C, 2, 1, WAVES, n_ff, (n_ff + WAVES / 2 - 1) / (WAVES / 2));
    const bool up = sc.part == 1;
    const gptr<uint8_t> Wg = (gptr<uint8_t>)W;
    // chunk m of the wave's row of output p; past the schedule the idle region
    auto load = [&](Q4Regs& r, const ItemCursor& it) {
        const int p = it.j < sc.tiles_wg ? sc.row(it.j) : sc.n;
        const int c = it.m;
        const bool real = p < sc.n && c < C;
        const bool last = c == C - 1;
        const int nbc = last ? nl : kChunkBlocks;
        const int sb = last ? sbl : 2 * kChunkBlocks;
        const int l = lane < nbc ? lane : nbc - 1;
        const int64_t row = real ? (int64_t)p + (up ? n_ff : 0) : 0;
        const gptr<uint8_t> cp = real ? Wg + row * row_bytes + (int64_t)c * kFullChunkBytesQ4 : idle_bytes();
        r.sc = load_u16<true>(cp + 2u * (uint32_t)l);
        r.a = load16<true>(cp + ((uint32_t)sb + 16u * (uint32_t)l));
    };
    auto compute = [&](const Q4Regs& r, int, int m, float& acc) {
        const int blk = m * kWave + lane;
        if (blk < NB) {
            const int s = q4_block_dot(r, m, lane, lds_q, lds_sx8);
            const float t = half_bits_to_float(r.sc) * lds_dx[blk];
            acc = __builtin_fmaf(t, (float)s, acc);
        }
    };
    Q4Regs R[kRingQ4];
    StageInput<ACT, WAVES * kWave> stage{xin, k, C, {}};
    stage.issue();
    __builtin_amdgcn_sched_barrier(0);
    ring_prologue(sc, R, load);
    __builtin_amdgcn_sched_barrier(0);
    stage.commit(lds_q, lds_dx, lds_res);
    __syncthreads();
    q4_block_sums<WAVES * kWave>(lds_q, lds_sx8, C);
    __syncthreads();
    if (sc.tiles_wg <= kKeepTiles) {
        // each wave keeps its row results in LDS and the pairs meet once,
        // after the row loop: no workgroup barrier inside the stream
        ring_loop(sc, R, load, compute, [&](float acc, int j, int, bool) {
            if (lane == 0) lds_res[j * WAVES + wave] = acc;
        });
        __syncthreads();
        for (int i = (int)threadIdx.x; i < sc.tiles_wg * sc.groups; i += WAVES * kWave) {
            const int j = i / sc.groups, grp = i % sc.groups;
            const int p = ((int)blockIdx.x + j * sc.grid) * sc.groups + grp;
            if (p < n_ff) {
                const float gate = lds_res[j * WAVES + 2 * grp], upv = lds_res[j * WAVES + 2 * grp + 1];
                // silu(g) u, as q8_i8_swiglu_kernel
                y[p] = gate / (1.0f + expf(-gate)) * upv;
            }
        }
        return;
    }
    ring_loop(sc, R, load, compute, [&](float acc, int, int p, bool valid) {
        // every wave ends each tile once: the pair meets in LDS
        if (lane == 0) lds_part[wave] = acc;
        __syncthreads();
        if (!up && valid && lane == 0) {
            const float gate = lds_part[wave], upv = lds_part[wave + 1];
            y[p] = gate / (1.0f + expf(-gate)) * upv;
        }
        __syncthreads();
    });
}

// The W4 GEMV with f32 activations (the W4A16 form of qwen3-8b-rtx4080-
// cutedsl, "W4A16 dequant-fused GEMM": 4-bit weights dequantized in
// registers against a wide activation): the f32 path's staging, ring and
// rotating split with a 4-bit item.  Each code word is turned into the
// int8 codes q = n - 8 exactly (per byte: set bit 7 so that subtracting 8
// cannot borrow from the next byte, then flip bit 7 back), so the block dot
// is the Q8_0 f32 path's, sum_i q_i x_i in f32 fused multiply-adds, then
// acc += d_w * that.
__device__ inline int q4_codes_i8(uint32_t nib) {
    return (int)(((nib | 0x80808080u) - 0x08080808u) ^ 0x80808080u);
}

template <int WAVES, int S>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(4)))
q4_f32_kernel(const uint8_t* __restrict__ W, int n, int k, const float* __restrict__ x, float* __restrict__ y) {
    static_assert(WAVES % S == 0, "S must divide WAVES");
    extern __shared__ __align__(16) uint8_t smem[];
    const int C = (int)chunk_count(k);
    const int NB = k / kBlock;
    const int nl = NB - (C - 1) * kChunkBlocks;
    const int sbl = (int)scale_section_bytes(nl);
    const int64_t row_bytes = q4_row_bytes(k);
    float4v* lds_x = reinterpret_cast<float4v*>(smem);
    float* lds_part = reinterpret_cast<float*>(smem + lds_f32act_bytes(C));
    float* lds_res = reinterpret_cast<float*>(smem + lds_f32act_bytes(C) + lds_tail_bytes<WAVES>());
    const int lane = threadIdx.x % kWave;
    const int wave = wave_id();
    const Sched sc(C, S, 1, WAVES, n, (n + WAVES / S - 1) / (WAVES / S));
    const gptr<uint8_t> Wg = (gptr<uint8_t>)W;
    // chunk c of a row (row n or chunk C: the idle region)
    auto load_rc = [&](Q4Regs& r, int row, int c) {
        const bool real = row < sc.n && c < C;
        const bool last = c == C - 1;
        const int nbc = last ? nl : kChunkBlocks;
        const int sb = last ? sbl : 2 * kChunkBlocks;
        const int l = lane < nbc ? lane : nbc - 1;
        const gptr<uint8_t> cp = real ? Wg + (int64_t)row * row_bytes + (int64_t)c * kFullChunkBytesQ4 : idle_bytes();
        r.sc = load_u16<true>(cp + 2u * (uint32_t)l);
        r.a = load16<true>(cp + ((uint32_t)sb + 16u * (uint32_t)l));
    };
    // word q of a block's 16 bytes: low nibbles are codes 4q..4q+3 (group q
    // of the staged activation), high nibbles codes 16+4q.. (group 4 + q)
    auto compute_c = [&](const Q4Regs& r, int c, float& acc) {
        if (c * kWave + lane < NB) {
            const float4v* xv = lds_x + (size_t)c * 8 * kWave + lane;
            int4v wa = r.a;
            opaque(wa);
            const uint32_t w4[4] = {(uint32_t)wa.x, (uint32_t)wa.y, (uint32_t)wa.z, (uint32_t)wa.w};
            float bs = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) bs = dot4_i8_f32(q4_codes_i8(w4[q] & 0x0F0F0F0Fu), xv[q * kWave], bs);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                bs = dot4_i8_f32(q4_codes_i8((w4[q] >> 4) & 0x0F0F0F0Fu), xv[(4 + q) * kWave], bs);
            acc = __builtin_fmaf(half_bits_to_float(r.sc), bs, acc);
        }
    };
    auto load = [&](Q4Regs& r, const ItemCursor& it) {
        load_rc(r, it.j < sc.tiles_wg ? sc.row(it.j) : sc.n, sc.chunk(it.m, 0));
    };
    auto compute = [&](const Q4Regs& r, int, int m, float& acc) { compute_c(r, sc.chunk(m, 0), acc); };
    constexpr bool kRot = S > 1;
    const bool rot = kRot && sc.tiles_wg <= kKeepTiles;
    RotSched rs;
    rs.set(sc, wave);
    auto rload = [&](Q4Regs& r, const RotSched& rs_, const RotCursor& it) {
        const bool has_item = it.j < rs_.sc->tiles_wg;
        load_rc(r, has_item ? sc.row(it.j) : sc.n, has_item ? it.p + S * it.m : C);
    };

    Q4Regs R[kRingQ4];
    StageF32<4, WAVES * kWave> st;
    st.issue(x, k);
    __builtin_amdgcn_sched_barrier(0);
    if (rot)
        rot_prologue(rs, R, rload);
    else
        ring_prologue(sc, R, load);
    __builtin_amdgcn_sched_barrier(0);
    st.commit(x, k, lds_x);
    __syncthreads();
    if constexpr (kRot) {
        if (rot) {
            if (threadIdx.x % kWave < (unsigned)sc.tiles_wg) {
                const int t = (int)(threadIdx.x % kWave);
                if (rs.items(t) == 0) lds_res[t * WAVES + sc.group * S + rs.part(t)] = 0.0f;
            }
            rot_loop(rs, R, rload,
                     [&](const Q4Regs& r, const Sched& s1, int, int m, float& acc) {
                         compute_c(r, s1.chunk(m, 0), acc);
                     },
                     [&](float acc, int t, int slot) {
                         if (lane == 0) lds_res[t * WAVES + slot] = acc;
                     });
            __syncthreads();
            flush_parts<WAVES>(sc, lds_res, y);
            return;
        }
    }
    uint64_t best = 0;
    ring_loop(sc, R, load, compute, [&](float acc, int, int row, bool) {
        finish_row<WAVES, S, false>(acc, row, n, lane, wave, lds_part, y, best);
    });
}

// The int8 path fed by the residual add + RMSNorm + re-quantization of
// residual_rmsnorm_q8_0, computed by every workgroup in its prologue
// (emit_qwen38_generate, "Where the speed comes from", item 3): the same
// codes and scales, bit for bit, with no launch of its own.
template <int WAVES, int S, int U>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(4)))
q8_i8_norm_kernel(const uint8_t* __restrict__ W, int n, int k, NormArgs na, float* __restrict__ y) {
    StageNorm<WAVES * kWave> stage{na, k, {}};
    q8_i8_body<WAVES, S, U, false, false>(W, n, k, y, nullptr, nullptr, stage);
}

// The dequantizing path's body; `stage` fills its f32 LDS layout
// (stage.issue() before the first weight items are requested,
// stage.commit(lds, unused, scratch) after).
template <int WAVES, int S, int U, bool ARGMAX, typename Stage>
__device__ __attribute__((always_inline)) inline void q8_f32_body(const uint8_t* __restrict__ W, int n, int k,
                                                                  float* __restrict__ y, uint64_t* __restrict__ keys,
                                                                  Stage& stage) {
    static_assert(WAVES % S == 0, "S must divide WAVES");
    extern __shared__ __align__(16) uint8_t smem[];
    const int C = (int)chunk_count(k);
    const int NB = k / kBlock;
    const int nl = NB - (C - 1) * kChunkBlocks;
    const int sbl = (int)scale_section_bytes(nl);
    const int64_t row_bytes = packed_row_bytes(k);
    float4v* lds_x = reinterpret_cast<float4v*>(smem);
    float* lds_part = reinterpret_cast<float*>(smem + lds_f32act_bytes(C));
    uint64_t* lds_key = reinterpret_cast<uint64_t*>(smem + ((lds_f32act_bytes(C) + WAVES * 4 + 15) & ~size_t(15)));
    const int lane = threadIdx.x % kWave;

    const Sched sc(C, S, U, WAVES, n, (n + WAVES / S - 1) / (WAVES / S));
    const gptr<uint8_t> Wg = (gptr<uint8_t>)W;
    auto load = [&](Q8Regs<U>& r, const ItemCursor& it) { q8_load_item<U>(r, Wg, row_bytes, sc, nl, sbl, it); };
    auto compute = [&](const Q8Regs<U>& r, int, int m, float& acc) { q8_f32_item<U>(r, sc, m, NB, lds_x, acc); };

    constexpr bool kRot = S > 1 && U == 1 && !ARGMAX;
    const int wave = wave_id();
    const bool rot = kRot && sc.tiles_wg <= kKeepTiles;
    float* lds_res = reinterpret_cast<float*>(smem + lds_f32act_bytes(C) + lds_tail_bytes<WAVES>());
    RotSched rs;
    rs.set(sc, wave);
    auto rload = [&](Q8Regs<1>& r, const RotSched& rs_, const RotCursor& it) {
        q8_load_rot(r, Wg, row_bytes, nl, sbl, rs_, it);
    };

    Q8Regs<U> R[kRingSets<U, S>];
    stage.issue();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kRot) {
        if (rot) {
            rot_prologue(rs, R, rload);
        } else {
            ring_prologue(sc, R, load);
        }
    } else {
        ring_prologue(sc, R, load);
    }
    __builtin_amdgcn_sched_barrier(0);
    stage.commit(reinterpret_cast<int4v*>(lds_x), nullptr, lds_res);
    __syncthreads();
    if constexpr (kRot) {
        if (rot) {
            if (threadIdx.x % kWave < (unsigned)sc.tiles_wg) {
                const int t = (int)(threadIdx.x % kWave);
                if (rs.items(t) == 0) lds_res[t * WAVES + sc.group * S + rs.part(t)] = 0.0f;
            }
            rot_loop(rs, R, rload,
                     [&](const Q8Regs<1>& r, const Sched& s1, int, int m, float& acc) {
                         q8_f32_item<1>(r, s1, m, NB, lds_x, acc);
                     },
                     [&](float acc, int t, int slot) {
                         if (lane == 0) lds_res[t * WAVES + slot] = acc;
                     });
            __syncthreads();
            flush_parts<WAVES>(sc, lds_res, y);
            return;
        }
    }
    uint64_t best = 0;
    ring_loop(sc, R, load, compute, [&](float acc, int, int row, bool) {
        finish_row<WAVES, S, ARGMAX>(acc, row, n, lane, wave, lds_part, y, best);
    });
    if constexpr (ARGMAX) write_block_key<WAVES>(best, lane, wave, lds_key, keys);
}

template <int WAVES, int S, int U, bool NT, bool ARGMAX>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(4)))
q8_f32_kernel(const uint8_t* __restrict__ W, int n, int k, const float* __restrict__ x, float* __restrict__ y,
              uint64_t* __restrict__ keys) {
    static_assert(NT, "the weight stream is always loaded non-temporally");
    StageInput<kActF32, WAVES * kWave> stage{x, k, (int)chunk_count(k), {}};
    q8_f32_body<WAVES, S, U, ARGMAX>(W, n, k, y, keys, stage);
}

// The dequantizing path fed by the residual add + RMSNorm of
// residual_rmsnorm_q8_0, computed by every workgroup in its prologue (the
// f32 form of q8_i8_norm_kernel, for deq 2): the staged values are that
// kernel's f32 output, bit for bit.
template <int WAVES, int S>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(4)))
q8_f32_norm_kernel(const uint8_t* __restrict__ W, int n, int k, NormArgs na, float* __restrict__ y) {
    StageNorm<WAVES * kWave, true> stage{na, k, {}};
    q8_f32_body<WAVES, S, 1, false>(W, n, k, y, nullptr, stage);
}

template <int WAVES, int S, int U, bool NT, bool ARGMAX>
__global__ void __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(4)))
bf16_kernel(const uint16_t* __restrict__ W, int n, int k, const float* __restrict__ x, float* __restrict__ y,
            uint64_t* __restrict__ keys) {
    static_assert(WAVES % S == 0, "S must divide WAVES");
    static_assert(NT, "the weight stream is always loaded non-temporally");
    extern __shared__ __align__(16) uint8_t smem[];
    const int C = bf16_chunks(k);
    float4v* lds_x = reinterpret_cast<float4v*>(smem);
    float* lds_part = reinterpret_cast<float*>(smem + lds_bf16_bytes(k));
    uint64_t* lds_key = reinterpret_cast<uint64_t*>(smem + ((lds_bf16_bytes(k) + WAVES * 4 + 15) & ~size_t(15)));
    const int lane = threadIdx.x % kWave;

    const Sched sc(C, S, U, WAVES, n, (n + WAVES / S - 1) / (WAVES / S));
    const gptr<uint16_t> Wg = (gptr<uint16_t>)W;
    auto load = [&](Bf16Regs<U>& r, const ItemCursor& it) { bf16_load_item<U>(r, Wg, k, sc, it); };
    auto compute = [&](const Bf16Regs<U>& r, int, int m, float& acc) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = sc.chunk(m, u);
            if (c < C) {
                const float4v* xv = lds_x + (size_t)c * 4 * kWave + lane;
                const int e0 = c * 1024 + 8 * lane;
                int4v wa = r.a[u], wb = r.b[u];
                opaque(wa);
                opaque(wb);
                if (e0 < k) acc = dot_bf16x8(wa, xv[0 * kWave], xv[1 * kWave], acc);
                if (e0 + 512 < k) acc = dot_bf16x8(wb, xv[2 * kWave], xv[3 * kWave], acc);
            }
        }
    };

    Bf16Regs<U> R[kRingSets<U, S>];
    StageBf16x<4, WAVES * kWave> st;
    st.issue(x, k);
    __builtin_amdgcn_sched_barrier(0);
    ring_prologue(sc, R, load);
    __builtin_amdgcn_sched_barrier(0);
    st.commit(x, k, lds_x);
    __syncthreads();
    uint64_t best = 0;
    const int wave = wave_id();
    ring_loop(sc, R, load, compute, [&](float acc, int, int row, bool) {
        finish_row<WAVES, S, ARGMAX>(acc, row, n, lane, wave, lds_part, y, best);
    });
    if constexpr (ARGMAX) write_block_key<WAVES>(best, lane, wave, lds_key, keys);
}

// ---------------------------------------------------------------- argmax
// Block sizes of the two argmax stages (compile-time, so no index waits
// for a load of the block size).
constexpr int kArgmax1Threads = 256, kArgmax2Threads = 1024;

__global__ void __launch_bounds__(kArgmax1Threads) argmax_stage1_kernel(const float* __restrict__ v, int64_t n,
                                                                         uint64_t* __restrict__ keys) {
    __shared__ uint64_t lds_key[16];
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t begin = (int64_t)blockIdx.x * per;
    const int64_t end = begin + per < n ? begin + per : n;
    uint64_t best = 0;
    for (int64_t i = begin + threadIdx.x; i < end; i += kArgmax1Threads) {
        const uint64_t key = argmax_key(v[i], (uint32_t)i);
        best = key > best ? key : best;
    }
    best = wave_max_u64(best);
    const int lane = threadIdx.x % kWave, wave = wave_id();
    if (lane == 0) lds_key[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t m = lds_key[0];
        for (int w = 1; w < kArgmax1Threads / kWave; ++w) m = lds_key[w] > m ? lds_key[w] : m;
        keys[blockIdx.x] = m;
    }
}

__global__ void __launch_bounds__(kArgmax2Threads) argmax_stage2_kernel(const uint64_t* __restrict__ keys, int count,
                                                                         int32_t* __restrict__ idx_out) {
    __shared__ uint64_t lds_key[16];
    uint64_t best = 0;
    for (int i = threadIdx.x; i < count; i += kArgmax2Threads) best = keys[i] > best ? keys[i] : best;
    best = wave_max_u64(best);
    const int lane = threadIdx.x % kWave, wave = wave_id();
    if (lane == 0) lds_key[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t m = lds_key[0];
        for (int w = 1; w < kArgmax2Threads / kWave; ++w) m = lds_key[w] > m ? lds_key[w] : m;
        idx_out[0] = (int32_t)argmax_key_index(m);
    }
}

// ------------------------------------------------------------- planning
constexpr int kMaxGrid = 8192;  // keys in the argmax workspace

// Per-device facts, looked up once per device (the device current at the
// call), so a process that drives several GPUs sizes each one's grids from
// that GPU.
constexpr int kMaxDevices = 64;
std::once_flag g_info_once[kMaxDevices];
DeviceInfo g_info[kMaxDevices];
DeviceInfo g_info_fallback;

int current_device() {
    int dev = 0;
    (void)hipGetDevice(&dev);
    return dev;
}

}  // namespace

const DeviceInfo& device_info() {
    const int dev = current_device();
    if (dev < 0 || dev >= kMaxDevices) {
        g_info_fallback.cus = 256;
        g_info_fallback.max_lds = 65536;
        return g_info_fallback;
    }
    std::call_once(g_info_once[dev], [dev] {
        DeviceInfo& d = g_info[dev];
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) d.cus = v;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess) d.max_lds = v;
        if (d.cus <= 0) d.cus = 256;
        if (d.max_lds <= 0) d.max_lds = 65536;
    });
    return g_info[dev];
}

namespace {

// Tuning overrides (0 = automatic): waves per row (split-K) and workgroups
// per CU.  Initialized from WSG_TUNE_SPLITK / WSG_TUNE_WG_PER_CU, changed at
// run time through wsg_tune().
int env_int(const char* name) {
    const char* v = std::getenv(name);
    return v ? std::atoi(v) : 0;
}

std::atomic<int> g_tune_splitk{-1};
std::atomic<int> g_tune_wg_per_cu{-1};
std::atomic<int> g_tune_waves{-1};
std::atomic<int> g_tune_unroll{-1};

int tune_read(std::atomic<int>& slot, const char* env) {
    int v = slot.load(std::memory_order_relaxed);
    if (v < 0) {
        v = env_int(env);
        slot.store(v, std::memory_order_relaxed);
    }
    return v;
}

int tune_waves() { return tune_read(g_tune_waves, "WSG_TUNE_WAVES"); }
int tune_unroll() { return tune_read(g_tune_unroll, "WSG_TUNE_UNROLL"); }

int tune_splitk() {
    int v = g_tune_splitk.load(std::memory_order_relaxed);
    if (v < 0) {
        v = env_int("WSG_TUNE_SPLITK");
        g_tune_splitk.store(v, std::memory_order_relaxed);
    }
    return v;
}

int tune_wg_per_cu() {
    int v = g_tune_wg_per_cu.load(std::memory_order_relaxed);
    if (v < 0) {
        v = env_int("WSG_TUNE_WG_PER_CU");
        g_tune_wg_per_cu.store(v, std::memory_order_relaxed);
    }
    return v;
}

// Workgroups resident per CU for a kernel with the given dynamic LDS
// (looked up once per device, kernel and LDS size).
template <typename K>
int resident_per_cu(K kernel, int threads, size_t lds) {
    static std::mutex mu;
    static std::map<std::tuple<int, const void*, size_t>, int> cache;
    const void* key = reinterpret_cast<const void*>(kernel);
    const auto id = std::make_tuple(current_device(), key, lds);
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(id);
    if (it != cache.end()) return it->second;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, key, threads, lds) != hipSuccess || blocks < 1)
        blocks = 1;
    cache[id] = blocks;
    return blocks;
}

// Persistent grid: at most (CUs x resident workgroups) workgroups, sized so
// that every workgroup walks the same number of row tiles (the last one at
// most as many).  A workgroup streams only a few GB/s, so one extra tile on
// some workgroups would stretch the whole launch by a tile's duration.
int persistent_grid(int tiles, int per_cu) {
    const int cus = device_info().cus;
    const int forced = tune_wg_per_cu();
    if (forced > 0 && forced < per_cu) per_cu = forced;
    int64_t gmax = (int64_t)cus * per_cu;
    if (gmax > kMaxGrid) gmax = kMaxGrid;
    if (tiles <= gmax) return tiles < 1 ? 1 : tiles;
    const int64_t rounds = (tiles + gmax - 1) / gmax;
    return (int)((tiles + rounds - 1) / rounds);
}

template <typename K>
void raise_lds_limit(K kernel, size_t lds) {
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
}

// Launch configuration of one GEMV call (reported by wsg_gemv_config).
struct LaunchInfo {
    int waves = 0, split = 0, unroll = 0, grid = 0;
    size_t lds = 0;
};

// kPathI8Gemv / kPathF32Gemv: the plain GEMV (and LM head) with int8 or f32
// activations; the fused norm and SwiGLU forms take kPathI8 / kPathF32.
enum Path { kPathI8 = 0, kPathF32 = 1, kPathBf16 = 2, kPathQ4 = 3, kPathQ4F32 = 4, kPathF32Gemv = 5, kPathI8Gemv = 6 };

// Default configuration per path and shape; tuning knobs override it.
struct Cfg {
    int waves, split, unroll;
};

// Waves per row for a Q8_0 GEMV, chosen so that the persistent token kernel
// (one 16-wave workgroup per CU, row tiles of 16/S rows dealt round robin)
// is balanced: cost = tiles per workgroup x the largest share of a row's
// chunks that one wave reads (the ragged last chunk counts by its blocks),
// with a 3% premium per doubling of S for the partial-sum exchange.  The
// eager kernels use the same factor, so both reduce a row in the same order
// and agree bit for bit.
int balanced_split(int64_t n, int64_t k) {
    const int64_t cus = device_info().cus > 0 ? device_info().cus : 1;
    const int64_t C = chunk_count(k);
    const double last = (double)last_chunk_blocks(k) / kChunkBlocks;
    int best = 1;
    double best_cost = 0.0;
    for (int S = 1, step = 0; S <= 4; S *= 2, ++step) {
        const int64_t rows_per_tile = 16 / S;
        const int64_t tiles = (n + rows_per_tile - 1) / rows_per_tile;
        const int64_t per_wg = (tiles + cus - 1) / cus;
        double part_max = 0.0;
        for (int p = 0; p < S; ++p) {
            double w = 0.0;
            for (int64_t c = p; c < C; c += S) w += (c == C - 1) ? last : 1.0;
            part_max = w > part_max ? w : part_max;
        }
        const double cost = (double)per_wg * part_max * (1.0 + 0.03 * step);
        if (S == 1 || cost < best_cost) {
            best = S;
            best_cost = cost;
        }
    }
    return best;
}

Cfg choose_cfg(Path path, int64_t n, int64_t k) {
    Cfg c;
    const int64_t rows_per_cu = n / device_info().cus;
    // measured on the 27B-stream shapes: 8-wave workgroups for tall
    // matrices; 16-wave workgroups (one per CU, a quarter of the staging
    // traffic) when there are few rows per CU
    c.waves = rows_per_cu < 32 ? 16 : 8;
    // one-chunk items, three in each wave's ring: measured fastest on every
    // workload shape once the ring's loads are pipelined
    c.unroll = 1;
    if (path == kPathQ4) {
        // measured on the 27B-stream shapes in 4 bits: 16-wave workgroups,
        // whole rows per wave (the per-workgroup staging is a larger share
        // of a 4-bit row) except long rows few per CU, which split in 4
        // (down: 13.6 against 14.8 us; qkvz, gate+up and out keep whole rows)
        c.waves = 16;
        c.split = (rows_per_cu < 32 && k >= 16384) ? 4 : 1;
    } else if (path == kPathQ4F32) {
        // measured on the same shapes with f32 activations (W4A16), where
        // the dequantizing arithmetic weighs more than the staging: 8-wave
        // workgroups, whole rows except long rows few per CU (down: split
        // 4); within 1% of the best of 4/8/16 waves x split 1/2/4 on all
        // four, up to 11% faster than 16 waves with whole rows
        c.waves = 8;
        c.split = (rows_per_cu < 32 && k >= 16384) ? 4 : 1;
    } else if (path == kPathBf16) {
        c.split = 1;
        if (rows_per_cu < 32 && k >= 16384) c.split = 4;
        else if (rows_per_cu < 8 && k >= 4096) c.split = 4;
        else if (rows_per_cu < 8 && k >= 2048) c.split = 2;
    } else {
        c.split = balanced_split(n, k);
        // the plain GEMV: 16-wave workgroups on every shape.  On the tall
        // 27B matrices they beat two 8-wave ones, with f32 activations
        // (deq 2: gate+up 32.5 against 33.7 us, qkvz 18.0 against 18.3) and
        // by less with int8 ones (the 27B token 4770 against 4792 us); the
        // LM head runs the same.  Not the fused norm and SwiGLU forms,
        // whose prologue and epilogue run slower at 16 waves.
        if (path == kPathF32Gemv || path == kPathI8Gemv) c.waves = 16;
    }
    const int tw = tune_waves(), ts = tune_splitk(), tu = tune_unroll();
    if (tw == 4 || tw == 8 || tw == 16) c.waves = tw;
    if (ts == 1 || ts == 2 || ts == 4) c.split = ts;
    if (tu == 1 || tu == 2 || tu == 4) c.unroll = tu;
    if (c.split > c.waves) c.split = c.waves;
    return c;
}

template <int V>
using IC = std::integral_constant<int, V>;

// Calls f(IC<waves>, IC<split>) for the compiled (waves, split) pairs.
template <typename F>
int dispatch_ws(int waves, int split, F&& f) {
    auto by_split = [&](auto W) -> int {
        switch (split) {
            case 2: return f(W, IC<2>{});
            case 4: return f(W, IC<4>{});
            default: return f(W, IC<1>{});
        }
    };
    switch (waves) {
        case 8: return by_split(IC<8>{});
        case 16: return by_split(IC<16>{});
        default: return by_split(IC<4>{});
    }
}

// Calls f(IC<waves>, IC<split>, IC<unroll>) with unroll from {1, 2, 4}
// (int8 and bf16 paths); the f32 path always loads one-chunk items (deeper
// unrolls exceed 128 VGPRs and spill).
template <bool F32, typename F>
int dispatch_wsu(int waves, int split, int unroll, F&& f) {
    return dispatch_ws(waves, split, [&](auto W, auto S) -> int {
        if constexpr (F32) {
            (void)unroll;
            return f(W, S, IC<1>{});
        } else {
            if (unroll <= 1) return f(W, S, IC<1>{});
            if (unroll == 2) return f(W, S, IC<2>{});
            return f(W, S, IC<4>{});
        }
    });
}

// Grid, LDS and (optionally) the launch of one kernel instantiation.
template <int WAVES, int S, typename K, typename... Args>
int launch_kernel(K kern, size_t lds, int n, LaunchInfo* info, int unroll, bool run, hipStream_t stream,
                  Args... args) {
    raise_lds_limit(kern, lds);
    const int tiles = (n + WAVES / S - 1) / (WAVES / S);
    const int grid = persistent_grid(tiles, resident_per_cu(kern, WAVES * kWave, lds));
    if (info) *info = LaunchInfo{WAVES, S, unroll, grid, lds};
    if (!run) return WSG_OK;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(WAVES * kWave), lds, stream, args...);
    return launch_status();
}

// The debug and argmax instantiations use the default one-chunk items (the
// unroll does not change the order of additions, so their results match the
// plain kernel at any unroll).
// Dynamic LDS of a Q8_0 kernel: the staged activation, the tail (split-K
// partials, argmax keys) and the kept partials of the rotating split path.
template <int WAVES>
size_t q8_lds_bytes(size_t lds_act) {
    return lds_act + lds_tail_bytes<WAVES>() + lds_keep_bytes<WAVES>();
}

template <int ACT, bool DEBUG, bool ARGMAX>
int launch_q8_i8(const void* w, int n, int k, const void* x, float* y, int32_t* dots, uint64_t* keys,
                 hipStream_t stream, LaunchInfo* info, bool run = true) {
    const Cfg c = choose_cfg(kPathI8Gemv, n, k);
    const size_t lds_act = lds_q8act_bytes((int)chunk_count(k));
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    if constexpr (DEBUG || ARGMAX) {
        return dispatch_ws(c.waves, c.split, [&](auto W, auto S) -> int {
            constexpr int Wv = decltype(W)::value, Sv = decltype(S)::value;
            auto kern = q8_i8_kernel<Wv, Sv, 1, ACT, true, DEBUG, ARGMAX>;
            return launch_kernel<Wv, Sv>(kern, q8_lds_bytes<Wv>(lds_act), n, info, 1, run, stream, wp, n, k,
                                         x, y, dots, keys);
        });
    } else {
        // four-chunk items with the requantizing staging exceed 128 VGPRs
        const int unroll = ACT == kActRequant && c.unroll > 2 ? 2 : c.unroll;
        return dispatch_wsu<false>(c.waves, c.split, unroll, [&](auto W, auto S, auto U) -> int {
            constexpr int Wv = decltype(W)::value, Sv = decltype(S)::value, Uv = decltype(U)::value;
            if constexpr (ACT == kActRequant && Uv > 2) {
                return WSG_ERR_MODE;  // never dispatched
            } else {
                auto kern = q8_i8_kernel<Wv, Sv, Uv, ACT, true, false, false>;
                return launch_kernel<Wv, Sv>(kern, q8_lds_bytes<Wv>(lds_act), n, info, Uv, run, stream, wp, n,
                                             k, x, y, dots, keys);
            }
        });
    }
}

// The int8 path fed by the fused residual + RMSNorm staging: the waves and
// split of the requantizing path for this shape, one-chunk items (the
// staging's registers leave no room for deeper ones).
int launch_q8_norm(const void* w, int n, int k, const NormArgs& na, float* y, hipStream_t stream, LaunchInfo* info,
                   bool run = true) {
    const Cfg c = choose_cfg(kPathI8, n, k);
    const size_t lds_act = lds_q8act_bytes((int)chunk_count(k));
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    return dispatch_ws(c.waves, c.split, [&](auto W, auto S) -> int {
        constexpr int Wv = decltype(W)::value, Sv = decltype(S)::value;
        auto kern = q8_i8_norm_kernel<Wv, Sv, 1>;
        return launch_kernel<Wv, Sv>(kern, q8_lds_bytes<Wv>(lds_act), n, info, 1, run, stream, wp, n, k, na, y);
    });
}

// The dequantizing path fed by the fused residual + RMSNorm staging (deq 2):
// the waves and split of the f32 path for this shape.
int launch_q8_norm_f32(const void* w, int n, int k, const NormArgs& na, float* y, hipStream_t stream,
                       LaunchInfo* info, bool run = true) {
    const Cfg c = choose_cfg(kPathF32, n, k);
    const size_t lds_act = lds_f32act_bytes((int)chunk_count(k));
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    return dispatch_ws(c.waves, c.split, [&](auto W, auto S) -> int {
        constexpr int Wv = decltype(W)::value, Sv = decltype(S)::value;
        auto kern = q8_f32_norm_kernel<Wv, Sv>;
        return launch_kernel<Wv, Sv>(kern, q8_lds_bytes<Wv>(lds_act), n, info, 1, run, stream, wp, n, k, na, y);
    });
}

// The W4 GEMV with the norm prologue: the W4 launch choice.
int launch_q4_norm(const void* w, int n, int k, const NormArgs& na, float* y, hipStream_t stream, LaunchInfo* info,
                   bool run = true) {
    const Cfg c = choose_cfg(kPathQ4, n, k);
    const size_t lds = lds_q8act_bytes((int)chunk_count(k));
    const size_t lds_sx8 = chunk_count(k) * kWave * 4;
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    return dispatch_ws(c.waves, c.split, [&](auto W, auto S) -> int {
        constexpr int Wv = decltype(W)::value, Sv = decltype(S)::value;
        auto kern = q4_i8_norm_kernel<Wv, Sv>;
        return launch_kernel<Wv, Sv>(kern, q8_lds_bytes<Wv>(lds) + lds_sx8, n, info, 1, run, stream, wp, n, k, na, y);
    });
}

// The 4-bit gate+up GEMV with the SwiGLU epilogue: the W4 waves, two per
// output (WAVES / 2 outputs per tile).
int launch_q4_swiglu(const void* w, int n_ff, int k, const void* x, int act_fmt, float* y, hipStream_t stream,
                     LaunchInfo* info, bool run = true) {
    const Cfg c = choose_cfg(kPathQ4, 2 * (int64_t)n_ff, k);
    const size_t lds = lds_q8act_bytes((int)chunk_count(k));
    const size_t lds_sx8 = chunk_count(k) * kWave * 4;
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    return dispatch_ws(c.waves, 1, [&](auto W, auto) -> int {
        constexpr int Wv = decltype(W)::value;
        if (act_fmt == WSG_ACT_Q8_0) {
            auto kern = q4_i8_swiglu_kernel<Wv, kActQ8>;
            return launch_kernel<Wv, 2>(kern, q8_lds_bytes<Wv>(lds) + lds_sx8, n_ff, info, 1, run, stream, wp, n_ff,
                                        k, x, y);
        }
        auto kern = q4_i8_swiglu_kernel<Wv, kActRequant>;
        return launch_kernel<Wv, 2>(kern, q8_lds_bytes<Wv>(lds) + lds_sx8, n_ff, info, 1, run, stream, wp, n_ff, k,
                                    x, y);
    });
}

// The W4 GEMV: its own waves and split choice (choose_cfg).
int launch_q4(const void* w, int n, int k, const void* x, int act_fmt, float* y, hipStream_t stream, LaunchInfo* info,
              bool run = true) {
    const Cfg c = choose_cfg(act_fmt == WSG_ACT_F32 ? kPathQ4F32 : kPathQ4, n, k);
    const size_t lds_act = lds_q8act_bytes((int)chunk_count(k));
    const size_t lds_sx8 = chunk_count(k) * kWave * 4;  // 8 sum x per block
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    return dispatch_ws(c.waves, c.split, [&](auto W, auto S) -> int {
        constexpr int Wv = decltype(W)::value, Sv = decltype(S)::value;
        if (act_fmt == WSG_ACT_F32) {
            auto kern = q4_f32_kernel<Wv, Sv>;
            const size_t lds = q8_lds_bytes<Wv>(lds_f32act_bytes((int)chunk_count(k)));
            return launch_kernel<Wv, Sv>(kern, lds, n, info, 1, run, stream, wp, n, k,
                                         static_cast<const float*>(x), y);
        }
        if (act_fmt == WSG_ACT_Q8_0) {
            auto kern = q4_i8_kernel<Wv, Sv, kActQ8>;
            return launch_kernel<Wv, Sv>(kern, q8_lds_bytes<Wv>(lds_act) + lds_sx8, n, info, 1, run, stream, wp, n,
                                         k, x, y);
        }
        auto kern = q4_i8_kernel<Wv, Sv, kActRequant>;
        return launch_kernel<Wv, Sv>(kern, q8_lds_bytes<Wv>(lds_act) + lds_sx8, n, info, 1, run, stream, wp, n, k,
                                     x, y);
    });
}

// The gate+up GEMV with the SwiGLU epilogue: the waves the int8 path
// uses for the whole gate+up matrix, one wave per output.
int launch_q8_swiglu(const void* w, int n_ff, int k, const void* x, int act_fmt, float* y, hipStream_t stream,
                     LaunchInfo* info, bool run = true) {
    const Cfg c = choose_cfg(act_fmt == WSG_ACT_F32 ? kPathF32 : kPathI8, 2 * (int64_t)n_ff, k);
    const size_t lds_act = act_fmt == WSG_ACT_F32 ? lds_f32act_bytes((int)chunk_count(k))
                                                  : lds_q8act_bytes((int)chunk_count(k));
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    return dispatch_ws(c.waves, 1, [&](auto W, auto) -> int {
        constexpr int Wv = decltype(W)::value;
        if (act_fmt == WSG_ACT_F32) {
            auto kern = q8_i8_swiglu_kernel<Wv, kActF32>;
            return launch_kernel<Wv, 1>(kern, q8_lds_bytes<Wv>(lds_act), n_ff, info, 1, run, stream, wp, n_ff, k, x,
                                        y);
        }
        if (act_fmt == WSG_ACT_Q8_0) {
            auto kern = q8_i8_swiglu_kernel<Wv, kActQ8>;
            return launch_kernel<Wv, 1>(kern, q8_lds_bytes<Wv>(lds_act), n_ff, info, 1, run, stream, wp, n_ff, k, x,
                                        y);
        }
        auto kern = q8_i8_swiglu_kernel<Wv, kActRequant>;
        return launch_kernel<Wv, 1>(kern, q8_lds_bytes<Wv>(lds_act), n_ff, info, 1, run, stream, wp, n_ff, k, x, y);
    });
}

template <bool ARGMAX>
int launch_q8_f32(const void* w, int n, int k, const float* x, float* y, uint64_t* keys, hipStream_t stream,
                  LaunchInfo* info, bool run = true) {
    const Cfg c = choose_cfg(kPathF32Gemv, n, k);
    const size_t lds_act = lds_f32act_bytes((int)chunk_count(k));
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    if constexpr (ARGMAX) {
        return dispatch_ws(c.waves, c.split, [&](auto W, auto S) -> int {
            constexpr int Wv = decltype(W)::value, Sv = decltype(S)::value;
            auto kern = q8_f32_kernel<Wv, Sv, 1, true, true>;
            return launch_kernel<Wv, Sv>(kern, q8_lds_bytes<Wv>(lds_act), n, info, 1, run, stream, wp, n, k,
                                         x, y, keys);
        });
    } else {
        return dispatch_wsu<true>(c.waves, c.split, c.unroll, [&](auto W, auto S, auto U) -> int {
            constexpr int Wv = decltype(W)::value, Sv = decltype(S)::value, Uv = decltype(U)::value;
            auto kern = q8_f32_kernel<Wv, Sv, Uv, true, false>;
            return launch_kernel<Wv, Sv>(kern, q8_lds_bytes<Wv>(lds_act), n, info, Uv, run, stream, wp, n, k,
                                         x, y, keys);
        });
    }
}

template <bool ARGMAX>
int launch_bf16(const uint16_t* w, int n, int k, const float* x, float* y, uint64_t* keys, hipStream_t stream,
                LaunchInfo* info, bool run = true) {
    const Cfg c = choose_cfg(kPathBf16, n, k);
    const size_t lds_act = lds_bf16_bytes(k);
    if constexpr (ARGMAX) {
        return dispatch_ws(c.waves, c.split, [&](auto W, auto S) -> int {
            constexpr int Wv = decltype(W)::value, Sv = decltype(S)::value;
            auto kern = bf16_kernel<Wv, Sv, 1, true, true>;
            return launch_kernel<Wv, Sv>(kern, lds_act + lds_tail_bytes<Wv>(), n, info, 1, run, stream, w, n, k, x,
                                         y, keys);
        });
    } else {
        return dispatch_wsu<false>(c.waves, c.split, c.unroll, [&](auto W, auto S, auto U) -> int {
            constexpr int Wv = decltype(W)::value, Sv = decltype(S)::value, Uv = decltype(U)::value;
            auto kern = bf16_kernel<Wv, Sv, Uv, true, false>;
            return launch_kernel<Wv, Sv>(kern, lds_act + lds_tail_bytes<Wv>(), n, info, Uv, run, stream, w, n, k, x,
                                         y, keys);
        });
    }
}

int launch_argmax_stage2(const uint64_t* keys, int count, int32_t* idx_out, hipStream_t stream) {
    hipLaunchKernelGGL(argmax_stage2_kernel, dim3(1), dim3(kArgmax2Threads), 0, stream, keys, count, idx_out);
    return launch_status();
}

int check_q8_args(const void* w, int64_t n, int64_t k, const void* x, int act_fmt, const void* out) {
    if (act_fmt != WSG_ACT_Q8_0 && act_fmt != WSG_ACT_F32 && act_fmt != WSG_ACT_F32_REQUANT) return WSG_ERR_MODE;
    if (n < 0 || k < 0 || n > kMaxDim || k > kMaxDim || k % kBlock) return WSG_ERR_SHAPE;
    const int64_t kmax = act_fmt == WSG_ACT_F32 ? WSG_MAX_K_F32ACT : WSG_MAX_K_Q8ACT;
    if (k > kmax) return WSG_ERR_SHAPE;
    if (n == 0) return WSG_OK;
    if (!out) return WSG_ERR_NULL;
    if (!aligned(out, 4)) return WSG_ERR_ALIGN;
    if (k == 0) return WSG_OK;
    if (!w || !x) return WSG_ERR_NULL;
    if (!aligned(w, 16) || !aligned(x, 16)) return WSG_ERR_ALIGN;
    return WSG_OK;
}

int check_bf16_args(const void* w, int64_t n, int64_t k, const void* x, const void* out) {
    if (n < 0 || k < 0 || n > kMaxDim || k > kMaxDim || k % 8) return WSG_ERR_SHAPE;
    if (k > WSG_MAX_K_F32ACT) return WSG_ERR_SHAPE;
    if (n == 0) return WSG_OK;
    if (!out) return WSG_ERR_NULL;
    if (!aligned(out, 4)) return WSG_ERR_ALIGN;
    if (k == 0) return WSG_OK;
    if (!w || !x) return WSG_ERR_NULL;
    if (!aligned(w, 16) || !aligned(x, 16)) return WSG_ERR_ALIGN;
    return WSG_OK;
}

}  // namespace

int gemv_split(bool f32_act, int64_t n, int64_t k) { return choose_cfg(f32_act ? kPathF32 : kPathI8, n, k).split; }

// Validation without launching (used by the plan).
int validate_gemv_q8(const void* w, int64_t n, int64_t k, const void* x, int act_fmt, const void* y) {
    return check_q8_args(w, n, k, x, act_fmt, y);
}

int validate_gemv_bf16(const void* w, int64_t n, int64_t k, const void* x, const void* y) {
    return check_bf16_args(w, n, k, x, y);
}

int validate_residual_rmsnorm(const float* h, const float* r, const float* g, int64_t k, float eps,
                              const void* h_out, const void* y, const void* y_q8);

namespace {
bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a && b && a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}
}  // namespace

int validate_gemv_q8_rmsnorm(const void* w, int64_t n, int64_t k, const float* h, const float* r, const float* g,
                             float eps, const void* h_out, const void* y, int act_fmt) {
    int rc = check_q8_args(w, n, k, h, act_fmt, y);
    if (rc != WSG_OK) return rc;
    if (n < 1 || k < kBlock) return WSG_ERR_SHAPE;
    rc = validate_residual_rmsnorm(h, r, g, k, eps, h_out, y, nullptr);
    if (rc != WSG_OK) return rc;
    // every workgroup reads h, r and g while workgroup 0 writes h_out
    if (overlaps(h_out, 4 * k, h, 4 * k) || overlaps(h_out, 4 * k, r, 4 * k) || overlaps(h_out, 4 * k, g, 4 * k) ||
        overlaps(y, 4 * n, h, 4 * k) || overlaps(y, 4 * n, r, 4 * k) || overlaps(y, 4 * n, g, 4 * k) ||
        overlaps(y, 4 * n, h_out, 4 * k))
        return WSG_ERR_MODE;
    return WSG_OK;
}

int validate_gemv_q4(const void* w, int64_t n, int64_t k, const void* x, int act_fmt, const void* y) {
    if (act_fmt != WSG_ACT_Q8_0 && act_fmt != WSG_ACT_F32_REQUANT && act_fmt != WSG_ACT_F32) return WSG_ERR_MODE;
    if (n < 1 || k < kBlock) return WSG_ERR_SHAPE;
    return check_q8_args(w, n, k, x, act_fmt, y);
}

int validate_gemv_q8_swiglu(const void* w, int64_t n_ff, int64_t k, const void* x, int act_fmt, const void* y) {
    if (act_fmt != WSG_ACT_Q8_0 && act_fmt != WSG_ACT_F32_REQUANT && act_fmt != WSG_ACT_F32) return WSG_ERR_MODE;
    if (n_ff < 1 || k < kBlock || 2 * n_ff > kMaxDim) return WSG_ERR_SHAPE;
    return check_q8_args(w, 2 * n_ff, k, x, act_fmt, y);
}

int validate_gemv_q4_swiglu(const void* w, int64_t n_ff, int64_t k, const void* x, int act_fmt, const void* y) {
    // the same arguments as the Q8_0 form (only the layout differs), int8 activations only
    if (act_fmt == WSG_ACT_F32) return WSG_ERR_MODE;
    return validate_gemv_q8_swiglu(w, n_ff, k, x, act_fmt, y);
}

namespace {
// Stage-1 workgroups (= argmax keys) of the LM-head launch of this shape on
// the current device; launches nothing.  -1 for an unknown format.
int lm_head_grid(int w_type, int act_fmt, int n, int k) {
    LaunchInfo info;
    int rc;
    if (w_type == WSG_W_BF16)
        rc = launch_bf16<true>(nullptr, n, k, nullptr, nullptr, nullptr, nullptr, &info, false);
    else if (act_fmt == WSG_ACT_F32)
        rc = launch_q8_f32<true>(nullptr, n, k, nullptr, nullptr, nullptr, nullptr, &info, false);
    else if (act_fmt == WSG_ACT_Q8_0)
        rc = launch_q8_i8<kActQ8, false, true>(nullptr, n, k, nullptr, nullptr, nullptr, nullptr, nullptr, &info,
                                                false);
    else if (act_fmt == WSG_ACT_F32_REQUANT)
        rc = launch_q8_i8<kActRequant, false, true>(nullptr, n, k, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                     &info, false);
    else
        return -1;
    return rc == WSG_OK ? info.grid : -1;
}

// The LM head's checks that do not involve the workspace.
int check_lm_head(const void* w, int w_type, int64_t n, int64_t k, const void* x, int act_fmt, const void* idx_out) {
    if (w_type != WSG_W_BF16 && w_type != WSG_W_Q8_0) return WSG_ERR_MODE;
    if (n < 1) return WSG_ERR_SHAPE;
    if (!idx_out) return WSG_ERR_NULL;
    if (!aligned(idx_out, 4)) return WSG_ERR_ALIGN;
    // logits pointer is optional: validate the GEMV part with a dummy non-null output
    const int rc = w_type == WSG_W_BF16 ? check_bf16_args(w, n, k, x, idx_out)
                                        : check_q8_args(w, n, k, x, act_fmt, idx_out);
    if (rc != WSG_OK) return rc;
    if (k == 0) return WSG_ERR_SHAPE;
    return WSG_OK;
}
}  // namespace

int validate_lm_head(const void* w, int w_type, int64_t n, int64_t k, const void* x, int act_fmt, const void* ws,
                     size_t ws_bytes, const void* idx_out) {
    int rc = check_lm_head(w, w_type, n, k, x, act_fmt, idx_out);
    if (rc != WSG_OK) return rc;
    if (!ws) return WSG_ERR_NULL;
    if (!aligned(ws, 8)) return WSG_ERR_ALIGN;
    const int grid = lm_head_grid(w_type, w_type == WSG_W_BF16 ? WSG_ACT_F32 : act_fmt, (int)n, (int)k);
    if (grid < 1) return WSG_ERR_HIP;
    if (ws_bytes < (size_t)grid * 8) return WSG_ERR_WORKSPACE;
    return WSG_OK;
}

// ------------------------------------------- the no-allocation LM head
// The stage-1 keys of lm_head_argmax_static: one array in the library's
// static device memory, kMaxGrid keys (64 KiB), which every GPU the library
// runs on holds until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device array: its device address is looked up
// with hipGetSymbolAddress, once per device with that device current, and
// only that address is passed to kernels.
namespace {
static __device__ __align__(256) uint64_t scratch[kMaxGrid];
constexpr size_t kScratchKeys = sizeof(scratch) / sizeof(scratch[0]);

std::mutex g_scratch_mu;
uint64_t* g_scratch_dev[kMaxDevices];  // device address of `scratch` per device (nullptr: not looked up)

// The current device's copy of `scratch` (looked up on the first call on
// that device).
int scratch_keys(uint64_t** out) {
    const int dev = current_device();
    if (dev < 0 || dev >= kMaxDevices) return WSG_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return WSG_ERR_HIP;
        }
        g_scratch_dev[dev] = static_cast<uint64_t*>(ptr);
    }
    *out = g_scratch_dev[dev];
    return WSG_OK;
}
}  // namespace

}  // namespace wsg

using namespace wsg;

extern "C" {

int gemv_q8_0(const void* w_packed, int64_t n, int64_t k, const void* x, int act_fmt, float* y,
              int32_t* debug_block_dots, hipStream_t stream) {
    int rc = check_q8_args(w_packed, n, k, x, act_fmt, y);
    if (rc != WSG_OK) return rc;
    if (debug_block_dots && act_fmt == WSG_ACT_F32) return WSG_ERR_MODE;
    if (debug_block_dots && !aligned(debug_block_dots, 4)) return WSG_ERR_ALIGN;
    if (n == 0) return WSG_OK;
    if (k == 0) return fill_zero_f32(y, n, stream);
    const int ni = (int)n, ki = (int)k;
    if (act_fmt == WSG_ACT_F32) return launch_q8_f32<false>(w_packed, ni, ki, static_cast<const float*>(x), y,
                                                            nullptr, stream, nullptr);
    if (act_fmt == WSG_ACT_Q8_0) {
        return debug_block_dots
                   ? launch_q8_i8<kActQ8, true, false>(w_packed, ni, ki, x, y, debug_block_dots, nullptr, stream,
                                                       nullptr)
                   : launch_q8_i8<kActQ8, false, false>(w_packed, ni, ki, x, y, nullptr, nullptr, stream, nullptr);
    }
    return debug_block_dots
               ? launch_q8_i8<kActRequant, true, false>(w_packed, ni, ki, x, y, debug_block_dots, nullptr, stream,
                                                        nullptr)
               : launch_q8_i8<kActRequant, false, false>(w_packed, ni, ki, x, y, nullptr, nullptr, stream, nullptr);
}

int gemv_q8_0_rmsnorm(const void* w_packed, int64_t n, int64_t k, const float* h, const float* r, const float* g,
                      float eps, float* h_out, float* y, hipStream_t stream) {
    const int rc = validate_gemv_q8_rmsnorm(w_packed, n, k, h, r, g, eps, h_out, y, WSG_ACT_F32_REQUANT);
    if (rc != WSG_OK) return rc;
    return launch_q8_norm(w_packed, (int)n, (int)k, NormArgs{h, r, g, h_out, eps}, y, stream, nullptr);
}

int gemv_q8_0_rmsnorm_f32(const void* w_packed, int64_t n, int64_t k, const float* h, const float* r,
                          const float* g, float eps, float* h_out, float* y, hipStream_t stream) {
    const int rc = validate_gemv_q8_rmsnorm(w_packed, n, k, h, r, g, eps, h_out, y, WSG_ACT_F32);
    if (rc != WSG_OK) return rc;
    return launch_q8_norm_f32(w_packed, (int)n, (int)k, NormArgs{h, r, g, h_out, eps}, y, stream, nullptr);
}

int gemv_q4_0_rmsnorm(const void* w_packed, int64_t n, int64_t k, const float* h, const float* r, const float* g,
                      float eps, float* h_out, float* y, hipStream_t stream) {
    // the same arguments and races as the Q8_0 form; only the weights differ
    const int rc = validate_gemv_q8_rmsnorm(w_packed, n, k, h, r, g, eps, h_out, y, WSG_ACT_F32_REQUANT);
    if (rc != WSG_OK) return rc;
    return launch_q4_norm(w_packed, (int)n, (int)k, NormArgs{h, r, g, h_out, eps}, y, stream, nullptr);
}

int gemv_q4_0_swiglu(const void* w_packed, int64_t n_ff, int64_t k, const void* x, int act_fmt, float* y,
                     hipStream_t stream) {
    const int rc = validate_gemv_q4_swiglu(w_packed, n_ff, k, x, act_fmt, y);
    if (rc != WSG_OK) return rc;
    return launch_q4_swiglu(w_packed, (int)n_ff, (int)k, x, act_fmt, y, stream, nullptr);
}

int gemv_q4_0(const void* w_packed, int64_t n, int64_t k, const void* x, int act_fmt, float* y, hipStream_t stream) {
    const int rc = validate_gemv_q4(w_packed, n, k, x, act_fmt, y);
    if (rc != WSG_OK) return rc;
    return launch_q4(w_packed, (int)n, (int)k, x, act_fmt, y, stream, nullptr);
}

int gemv_q8_0_swiglu(const void* w_packed, int64_t n_ff, int64_t k, const void* x, int act_fmt, float* y,
                     hipStream_t stream) {
    const int rc = validate_gemv_q8_swiglu(w_packed, n_ff, k, x, act_fmt, y);
    if (rc != WSG_OK) return rc;
    return launch_q8_swiglu(w_packed, (int)n_ff, (int)k, x, act_fmt, y, stream, nullptr);
}

int gemv_bf16(const uint16_t* w, int64_t n, int64_t k, const float* x, float* y, hipStream_t stream) {
    int rc = check_bf16_args(w, n, k, x, y);
    if (rc != WSG_OK) return rc;
    if (n == 0) return WSG_OK;
    if (k == 0) return fill_zero_f32(y, n, stream);
    return launch_bf16<false>(w, (int)n, (int)k, x, y, nullptr, stream, nullptr);
}

int64_t wsg_argmax_ws_bytes(void) { return (int64_t)kMaxGrid * 8; }

int64_t lm_head_argmax_ws_bytes(int64_t n, int64_t k, int w_type) {
    if (w_type != WSG_W_BF16 && w_type != WSG_W_Q8_0) return -1;
    if (n < 1 || k < 1 || n > kMaxDim || k > kMaxDim) return -1;
    if (w_type == WSG_W_BF16 ? (k % 8 || k > WSG_MAX_K_F32ACT) : (k % kBlock || k > WSG_MAX_K_Q8ACT)) return -1;
    int grid = 0;
    if (w_type == WSG_W_BF16) {
        grid = lm_head_grid(WSG_W_BF16, WSG_ACT_F32, (int)n, (int)k);
    } else {
        // every activation format of the Q8_0 head (the f32 one only where k allows it)
        for (int act : {WSG_ACT_Q8_0, WSG_ACT_F32_REQUANT, WSG_ACT_F32}) {
            if (act == WSG_ACT_F32 && k > WSG_MAX_K_F32ACT) continue;
            const int g = lm_head_grid(WSG_W_Q8_0, act, (int)n, (int)k);
            if (g < 1) return -1;
            grid = g > grid ? g : grid;
        }
    }
    return grid < 1 ? -1 : (int64_t)grid * 8;
}

int wsg_tune(int knob, int value) {
    if (value < 0) return WSG_ERR_SHAPE;
    switch (knob) {
        case WSG_TUNE_SPLITK:
            if (value != 0 && value != 1 && value != 2 && value != 4) return WSG_ERR_SHAPE;
            g_tune_splitk.store(value);
            return WSG_OK;
        case WSG_TUNE_WG_PER_CU:
            g_tune_wg_per_cu.store(value);
            return WSG_OK;
        case WSG_TUNE_WAVES:
            if (value != 0 && value != 4 && value != 8 && value != 16) return WSG_ERR_SHAPE;
            g_tune_waves.store(value);
            return WSG_OK;
        case WSG_TUNE_UNROLL:
            if (value != 0 && value != 1 && value != 2 && value != 4) return WSG_ERR_SHAPE;
            g_tune_unroll.store(value);
            return WSG_OK;
        default: return WSG_ERR_MODE;
    }
}

int wsg_gemv_config(int w_type, int act_fmt, int64_t n, int64_t k, int* waves, int* split, int* unroll,
                    int* grid, int64_t* lds_bytes) {
    if (w_type != WSG_W_BF16 && w_type != WSG_W_Q8_0) return WSG_ERR_MODE;
    if (w_type == WSG_W_BF16) act_fmt = WSG_ACT_F32;
    if (act_fmt != WSG_ACT_Q8_0 && act_fmt != WSG_ACT_F32 && act_fmt != WSG_ACT_F32_REQUANT) return WSG_ERR_MODE;
    if (n < 1 || k < 1 || n > kMaxDim || k > kMaxDim) return WSG_ERR_SHAPE;
    if (w_type == WSG_W_BF16 ? (k % 8 || k > WSG_MAX_K_F32ACT)
                             : (k % kBlock || k > (act_fmt == WSG_ACT_F32 ? WSG_MAX_K_F32ACT : WSG_MAX_K_Q8ACT)))
        return WSG_ERR_SHAPE;
    LaunchInfo info;
    const int ni = (int)n, ki = (int)k;
    int rc;
    if (w_type == WSG_W_BF16)
        rc = launch_bf16<false>(nullptr, ni, ki, nullptr, nullptr, nullptr, nullptr, &info, false);
    else if (act_fmt == WSG_ACT_F32)
        rc = launch_q8_f32<false>(nullptr, ni, ki, nullptr, nullptr, nullptr, nullptr, &info, false);
    else if (act_fmt == WSG_ACT_Q8_0)
        rc = launch_q8_i8<kActQ8, false, false>(nullptr, ni, ki, nullptr, nullptr, nullptr, nullptr, nullptr, &info,
                                                false);
    else
        rc = launch_q8_i8<kActRequant, false, false>(nullptr, ni, ki, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                     &info, false);
    if (rc != WSG_OK) return rc;
    if (waves) *waves = info.waves;
    if (split) *split = info.split;
    if (unroll) *unroll = info.unroll;
    if (grid) *grid = info.grid;
    if (lds_bytes) *lds_bytes = (int64_t)info.lds;
    return WSG_OK;
}

namespace {
// The LM-head GEMV with stage 1 into `keys`, then stage 2 (arguments checked).
int launch_lm_head(const void* w, int w_type, int64_t n, int64_t k, const void* x, int act_fmt, uint64_t* keys,
                   int32_t* idx_out, float* debug_logits, hipStream_t stream) {
    int rc;
    const int ni = (int)n, ki = (int)k;
    LaunchInfo info;
    if (w_type == WSG_W_BF16) {
        rc = launch_bf16<true>(static_cast<const uint16_t*>(w), ni, ki, static_cast<const float*>(x), debug_logits,
                               keys, stream, &info);
    } else if (act_fmt == WSG_ACT_F32) {
        rc = launch_q8_f32<true>(w, ni, ki, static_cast<const float*>(x), debug_logits, keys, stream, &info);
    } else if (act_fmt == WSG_ACT_Q8_0) {
        rc = launch_q8_i8<kActQ8, false, true>(w, ni, ki, x, debug_logits, nullptr, keys, stream, &info);
    } else {
        rc = launch_q8_i8<kActRequant, false, true>(w, ni, ki, x, debug_logits, nullptr, keys, stream, &info);
    }
    if (rc != WSG_OK) return rc;
    return launch_argmax_stage2(keys, info.grid, idx_out, stream);
}
}  // namespace

int lm_head_argmax(const void* w, int w_type, int64_t n, int64_t k, const void* x, int act_fmt, void* ws,
                   size_t ws_bytes, int32_t* idx_out, float* debug_logits, hipStream_t stream) {
    const int rc = validate_lm_head(w, w_type, n, k, x, act_fmt, ws, ws_bytes, idx_out);
    if (rc != WSG_OK) return rc;
    if (debug_logits && !aligned(debug_logits, 4)) return WSG_ERR_ALIGN;
    return launch_lm_head(w, w_type, n, k, x, act_fmt, static_cast<uint64_t*>(ws), idx_out, debug_logits, stream);
}

int lm_head_argmax_static(const void* w, int w_type, int64_t n, int64_t k, const void* x, int act_fmt,
                          int32_t* idx_out, float* debug_logits, hipStream_t stream) {
    int rc = check_lm_head(w, w_type, n, k, x, act_fmt, idx_out);
    if (rc != WSG_OK) return rc;
    if (debug_logits && !aligned(debug_logits, 4)) return WSG_ERR_ALIGN;
    // the stage-1 keys must fit the static array (the grid never exceeds
    // kMaxGrid workgroups, so every valid shape does)
    const int grid = lm_head_grid(w_type, w_type == WSG_W_BF16 ? WSG_ACT_F32 : act_fmt, (int)n, (int)k);
    if (grid < 1) return WSG_ERR_HIP;
    if ((size_t)grid > kScratchKeys) return WSG_ERR_WORKSPACE;
    uint64_t* keys = nullptr;
    rc = scratch_keys(&keys);
    if (rc != WSG_OK) return rc;
    return launch_lm_head(w, w_type, n, k, x, act_fmt, keys, idx_out, debug_logits, stream);
}

int argmax_f32(const float* v, int64_t n, void* ws, size_t ws_bytes, int32_t* idx_out, hipStream_t stream) {
    if (n < 1 || n > kMaxDim) return WSG_ERR_SHAPE;
    if (!v || !ws || !idx_out) return WSG_ERR_NULL;
    if (!aligned(v, 4) || !aligned(ws, 8) || !aligned(idx_out, 4)) return WSG_ERR_ALIGN;
    if (ws_bytes < (size_t)kMaxGrid * 8) return WSG_ERR_WORKSPACE;
    int64_t g = (n + 4095) / 4096;
    const int64_t cap = (int64_t)device_info().cus * 4;
    if (g > cap) g = cap;
    if (g > kMaxGrid) g = kMaxGrid;
    if (g < 1) g = 1;
    uint64_t* keys = static_cast<uint64_t*>(ws);
    hipLaunchKernelGGL(argmax_stage1_kernel, dim3((unsigned)g), dim3(kArgmax1Threads), 0, stream, v, n, keys);
    int rc = launch_status();
    if (rc != WSG_OK) return rc;
    return launch_argmax_stage2(keys, (int)g, idx_out, stream);
}

}  // extern "C"

#ifdef WSG_TIMELINE
// Diagnostic build only: where the GEMV kernels' workgroups record their
// timestamps (timeline.hpp); buf = nullptr stops recording.
extern "C" __attribute__((visibility("default"))) int wsg_timeline_set(void* buf, uint32_t modulus) {
    if (wsg::tl_set_here(buf, modulus) != 0 || wsg::stream_timeline_set(buf, modulus) != 0) return WSG_ERR_HIP;
    return WSG_OK;
}
#endif
