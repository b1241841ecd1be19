/* wsgemv -- batch-1 decode GEMV weight streaming on MI355X (gfx950).
 *
 * The operation (emit_qwen38_generate, "Where the speed comes from"): at
 * batch 1 a decode step is bandwidth-bound; each projection is one GEMV
 * y = W.x that streams a whole weight matrix against ONE activation vector.
 * Projections that share an activation are stacked by rows into one matrix
 * (q/k/v/z, gate+up), so each is one launch (item 1).  Weights are BF16 or
 * Q8_0 blocks (32 int8 codes + one fp16 scale, llama.cpp style).  The
 * activation is either quantized to int8 per 32-block, so the inner loop is
 * an int8 dot product, or kept in f32 and the weights are dequantized in
 * registers (the "deq" modes 0/1/2 of the same page).  The step ends with
 * an LM-head GEMV whose argmax stays on the device (item 2; GPU Kernel Lab,
 * "Decode integration").
 *
 * Conventions for every entry point:
 *  - Every pointer argument is a DEVICE pointer (except the descriptor array
 *    of the plan calls and the outputs of the size and config queries,
 *    which are host memory), allocated and owned by the caller.
 *  - The hot calls (quantizers, GEMVs, the norm step, the LM head, embedding
 *    and advance, the probes) allocate no device memory, never synchronize
 *    the host with the device and can be captured into a hipGraph.  The
 *    exceptions, which must not be called while a stream is capturing:
 *    wsg_plan_create (builds and instantiates a graph, host memory only),
 *    wsg_plan_create_persistent (allocates device state and synchronizes
 *    the device), wsg_plan_error / wsg_plan_error_detail (synchronize),
 *    wsg_plan_destroy (frees), and the first lm_head_argmax_static call on
 *    each device (looks up its static array; later calls are capturable).
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *    The return value is a status code, decided BEFORE anything is
 *    enqueued: on any nonzero status nothing was launched.  WSG_ERR_HIP
 *    reports a launch that the runtime rejected.  Faults inside a kernel
 *    surface at the caller's next synchronization, as usual in HIP.
 *  - Outputs are overwritten, never accumulated into.
 *  - Weight, activation and quantized-activation pointers must be 16-byte
 *    aligned; f32 outputs and int32 outputs 4-byte aligned.
 *  - Sizes are int64_t (signed, so that the size queries can return -1 for
 *    a bad shape); n and k must each be < 2^31.
 *  - State: the library looks up per-device launch parameters once per
 *    device (the device current at the call); wsg_tune holds process-wide
 *    tuning knobs (for measurement sweeps) that change the launch shape of
 *    later calls from every thread; lm_head_argmax_static keeps one static
 *    array per GPU.  Apart from wsg_tune and overlapping calls of
 *    lm_head_argmax_static on one GPU, all entry points are thread-safe.
 */
#ifndef WSGEMV_H
#define WSGEMV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; everything declared here is
 * exported. */
#pragma GCC visibility push(default)

/* ---------------------------------------------------------------- status */
enum {
    WSG_OK = 0,
    WSG_ERR_NULL = 1,      /* a required pointer is NULL */
    WSG_ERR_SHAPE = 2,     /* n/k out of range, k not a multiple of the block */
    WSG_ERR_ALIGN = 3,     /* a pointer violates the alignment rule above */
    WSG_ERR_MODE = 4,      /* unknown activation format / weight type / op */
    WSG_ERR_WORKSPACE = 5, /* workspace too small */
    WSG_ERR_HIP = 6,       /* the HIP runtime rejected a call */
};

/* Activation formats of the Q8_0 GEMV (the deq modes of emit_qwen38_generate):
 *  WSG_ACT_Q8_0        x is the output of quantize_act_q8_0: int8 dot path.
 *  WSG_ACT_F32_REQUANT x is f32[k]; each workgroup quantizes it with the same
 *                      rule and the same bytes as quantize_act_q8_0, then
 *                      takes the int8 dot path (one launch instead of two).
 *  WSG_ACT_F32         x is f32[k]: the dequantizing path, no activation
 *                      quantization error.
 * deq 0 -> every Q8_0 GEMV uses WSG_ACT_Q8_0 (or _F32_REQUANT);
 * deq 1 -> the same, except the LM head uses WSG_ACT_F32;
 * deq 2 -> every Q8_0 GEMV uses WSG_ACT_F32.  BF16 GEMVs always take f32 x. */
enum { WSG_ACT_Q8_0 = 0, WSG_ACT_F32 = 1, WSG_ACT_F32_REQUANT = 2 };

/* Weight types. */
enum { WSG_W_BF16 = 0, WSG_W_Q8_0 = 1 };

/* Largest supported k per path (the activation is staged whole in LDS). */
#define WSG_MAX_K_Q8ACT 57344 /* WSG_ACT_Q8_0 and WSG_ACT_F32_REQUANT */
#define WSG_MAX_K_F32ACT 36864 /* WSG_ACT_F32 and BF16 weights */

/* Static text for a status code (never NULL). */
const char* wsg_status_str(int status);

/* Library version, "major.minor.patch". */
const char* wsg_version(void);

/* ---------------------------------------------------------- Q8_0 layout ---
 * Canonical interchange (llama.cpp block order): per row, per 32 weights
 * along k, a 34-byte block {fp16 scale d (little-endian); int8 q[32]};
 * weight = d * q.
 *
 * Device layout ("packed"), produced only by pack_q8_0 or
 * quantize_q8_0_weights: rows are contiguous, row r at byte
 * r * q8_0_row_bytes(k).  A row is split into chunks of up to 64 blocks
 * (2048 weights); a chunk of nb blocks holds
 *     [nb fp16 scales, zero-padded to a multiple of 16 bytes]
 *     [first 16 codes of each of its nb blocks, 16 bytes per block]
 *     [last 16 codes of each of its nb blocks]
 * so one wave of 64 lanes loads one whole block per lane with two
 * contiguous 1 KB loads.  Bytes per weight stay 34/32 whenever k % 256 == 0
 * (otherwise the last chunk carries up to 14 bytes of padding).
 */
int64_t q8_0_row_bytes(int64_t k);
int64_t q8_0_packed_bytes(int64_t n, int64_t k);

/* ------------------------------------------------ offline weight prep ---
 * Concatenation of projections that share an activation = writing each
 * projection's rows into consecutive row ranges of one packed matrix:
 * pass w_packed + row0 * q8_0_row_bytes(k) (resp. out + row0 * k).
 */

/* Canonical AoS blocks (n rows x k/32 blocks x 34 bytes, any alignment)
 * -> device layout.  k % 32 == 0. */
int pack_q8_0(const void* blocks_aos, int64_t n, int64_t k, void* w_packed, hipStream_t stream);

/* Row-major f32 weights [n][k] -> device layout, with the Q8_0 rule:
 * d = fp16_RNE(max|w| / 127) (IEEE fp32 divide), q = clamp(round half away
 * from zero of w / float(d), -127, 127) (fp32 divide by the stored scale);
 * an all-zero block (or one whose scale underflows fp16) stores d = +0,
 * q = 0.  Non-finite weights are outside the contract.  k % 32 == 0. */
int quantize_q8_0_weights(const float* w, int64_t n, int64_t k, void* w_packed, hipStream_t stream);

/* f32 -> bf16, round to nearest even, count elements. */
int convert_bf16(const float* in, int64_t count, uint16_t* out, hipStream_t stream);

/* ------------------------------------------ activation quantization ---
 * x f32[k] -> planar Q8_0 activation: int8 q[k] at byte 0, then fp16
 * d[k/32] at byte k (natural order, same rule as quantize_q8_0_weights).
 * k % 32 == 0.  act_q8_0_bytes(k) = k + k/16. */
int64_t act_q8_0_bytes(int64_t k);
int quantize_act_q8_0(const float* x, int64_t k, void* x_q8, hipStream_t stream);

/* ------------------------------------ residual add + RMSNorm + requant ---
 * The step either side of every GEMV of a decode layer, in one kernel
 * (emit_qwen38_generate, "Where the speed comes from", item 3: the residual
 * add, the next RMSNorm and the activation re-quantization; GPU Kernel Lab,
 * "Decode integration": FP32 reduction, residual fusion):
 *     h'_i = h_i + r_i                      (one fp32 add; r NULL: h' = h)
 *     y_i  = h'_i * s * g_i,  s = 1 / sqrt(mean_j h'_j^2 + eps)
 *                                           (fp32; g NULL: gain 1)
 *     y_q8 = the planar Q8_0 activation of y, exactly as quantize_act_q8_0
 *            would write it from the f32 y (act_q8_0_bytes(k) bytes).
 * h, r, g are f32[k]; h_out (h'), y (f32[k]) and y_q8 are outputs, each
 * optional (NULL: not written; all three NULL: nothing is launched).  h_out
 * may be h or r (an in-place residual update); no other buffers may overlap.
 * k % 32 == 0, k <= WSG_MAX_K_Q8ACT; eps finite and > 0, else WSG_ERR_MODE.
 * The mean of squares is accumulated in fp32 in a fixed order, so results
 * repeat bit for bit.  One workgroup (the vector is small; the call is
 * latency-bound).  Acceptance: h_out bit-exact (one IEEE add);
 * |y - y_ref| <= 2^-16 |y_ref| against the fp64 definition;
 * y_q8 bit-exact against the Q8_0 rule applied to the y this call computes. */
int residual_rmsnorm_q8_0(const float* h, const float* r, const float* g, int64_t k, float eps, float* h_out,
                          float* y, void* y_q8, hipStream_t stream);

/* The int8-activation Q8_0 GEMV fed by residual_rmsnorm_q8_0, which every
 * workgroup computes in its prologue instead of a launch of its own
 * (emit_qwen38_generate, "Where the speed comes from", item 3):
 *   h' = h + r (r nullable), x = h' / sqrt(mean h'^2 + eps) * g (g nullable),
 *   y = W . Q8_0(x)  (int8 activations, as gemv_q8_0 with WSG_ACT_Q8_0),
 * and h' is written to h_out (nullable) by one workgroup.  The mean of
 * squares is reduced in the order residual_rmsnorm_q8_0 uses and the codes
 * are computed with the same operations, so y equals gemv_q8_0 fed that
 * call's y_q8, bit for bit, and h_out equals its h_out.  W in the device
 * layout, n >= 1, 32 <= k <= WSG_MAX_K_Q8ACT, k % 32 == 0 (WSG_ERR_SHAPE);
 * eps as for residual_rmsnorm_q8_0 (WSG_ERR_MODE); h, r, g, h_out 16-byte
 * aligned; h_out must not overlap h, r or g, and y must overlap none of
 * h, r, g, h_out (WSG_ERR_MODE): other workgroups still read the inputs
 * while one writes h_out. */
int gemv_q8_0_rmsnorm(const void* w_packed, int64_t n, int64_t k, const float* h, const float* r, const float* g,
                      float eps, float* h_out, float* y, hipStream_t stream);

/* The deq 2 form of gemv_q8_0_rmsnorm: the same residual add + RMSNorm in
 * every workgroup's prologue, then the dequantizing GEMV on the f32
 * normalized vector (no activation quantization; emit_qwen38_generate,
 * "Where the speed comes from", the deq paragraph):
 *   y = W . (h' / sqrt(mean h'^2 + eps) * g),  f32 activations,
 * bit for bit gemv_q8_0 with WSG_ACT_F32 fed the y (f32) that
 * residual_rmsnorm_q8_0 computes, and h_out as that call's h_out.
 * Arguments, races and errors as gemv_q8_0_rmsnorm, with
 * 32 <= k <= WSG_MAX_K_F32ACT. */
int gemv_q8_0_rmsnorm_f32(const void* w_packed, int64_t n, int64_t k, const float* h, const float* r,
                          const float* g, float eps, float* h_out, float* y, hipStream_t stream);

/* ---------------------------------------------------------- W4 weights --
 * 4-bit blocks (qwen3-8b-rtx4080-cutedsl, "W4A16 dequant-fused GEMM"; GPU
 * Kernel Lab, "Quantization experiments"): per 32 weights an fp16 scale
 * d = fp16(max|w| / 7) and codes q = clamp(round(w / d), -7, 7) (the fp32
 * quotient by the stored scale, half away from zero), stored as q + 8 in
 * 4 bits: 18 bytes per block, 0.5625 bytes per weight.  Device layout: rows
 * of q4_0_row_bytes(k) bytes; per 2048-weight chunk [64 fp16 scales][64 x
 * 16 code bytes], a block's byte j holding code j (low nibble) and code
 * j + 16 (high nibble); the last chunk's scale section is padded to 16
 * bytes with zeros.  q4_0_*_bytes return -1 on a bad shape.
 * gemv_q4_0: y = W x.  With int8 activations (act_fmt WSG_ACT_Q8_0 or
 *   WSG_ACT_F32_REQUANT) the exact int32 block dot s = sum q_w q_x, then
 *   y = sum_b d_w d_x s in f32, accepted as gemv_q8_0's int8 path,
 *   32 <= k <= WSG_MAX_K_Q8ACT.  With f32 activations (WSG_ACT_F32, the
 *   W4A16 form of qwen3-8b-rtx4080-cutedsl, "W4A16 dequant-fused GEMM")
 *   y = sum_b d_w sum_i q_i x_i in f32 fused multiply-adds, accepted as
 *   gemv_q8_0's f32 path, 32 <= k <= WSG_MAX_K_F32ACT.  Other act_fmt:
 *   WSG_ERR_MODE; n >= 1 and k % 32 == 0 else WSG_ERR_SHAPE.
 * The "q4_0" names say "4-bit, block of 32, one scale" only: these blocks
 * are NOT llama.cpp's Q4_0 (whose scale is signed and whose codes span
 * [-8, 7]); llama.cpp Q4_0 files cannot be loaded through them. */
int64_t q4_0_row_bytes(int64_t k);
int64_t q4_0_packed_bytes(int64_t n, int64_t k);
int quantize_q4_0_weights(const float* w, int64_t n, int64_t k, void* w_packed, hipStream_t stream);
int gemv_q4_0(const void* w_packed, int64_t n, int64_t k, const void* x, int act_fmt, float* y, hipStream_t stream);

/* gemv_q4_0_rmsnorm: the 4-bit GEMV fed by the residual add + RMSNorm +
 * re-quantization of residual_rmsnorm_q8_0 computed in its own prologue
 * (emit_qwen38_generate, "Where the speed comes from", item 3, on 4-bit
 * weights): y = W . Q8_0(RMSNorm(h + r) * g), bit for bit the output of
 * residual_rmsnorm_q8_0 followed by gemv_q4_0 with WSG_ACT_Q8_0 on its
 * codes.  Arguments, h_out, acceptance and errors as gemv_q8_0_rmsnorm,
 * with w_packed in the 4-bit layout above. */
int gemv_q4_0_rmsnorm(const void* w_packed, int64_t n, int64_t k, const float* h, const float* r, const float* g,
                      float eps, float* h_out, float* y, hipStream_t stream);

/* gemv_q4_0_swiglu: the 4-bit gate+up GEMV with the SwiGLU epilogue (GPU
 * Kernel Lab, "What we built", "Decode integration", on 4-bit weights):
 * w_packed holds 2 n_ff rows in the 4-bit layout, gate rows first;
 * y[p] = silu(g_p) u_p with g_p, u_p the int8-path outputs of rows p and
 * n_ff + p.  Arguments, acceptance and errors as gemv_q8_0_swiglu, with
 * int8 activations only (WSG_ACT_F32: WSG_ERR_MODE). */
int gemv_q4_0_swiglu(const void* w_packed, int64_t n_ff, int64_t k, const void* x, int act_fmt, float* y,
                     hipStream_t stream);

/* The gate+up GEMV with its SwiGLU epilogue (GPU Kernel Lab, "What we
 * built", "Decode integration": the dual gate/up projection fused with
 * SwiGLU at batch 1):
 *   g_p = W[p] . x,  u_p = W[n_ff + p] . x,  y[p] = silu(g_p) u_p,
 *   silu(t) = t / (1 + exp(-t)),  p < n_ff,
 * for W in the device layout with 2 n_ff rows (the concatenated gate+up
 * matrix, gate rows first), with int8 activations (act_fmt WSG_ACT_Q8_0 or
 * WSG_ACT_F32_REQUANT) or f32 ones (WSG_ACT_F32: the W8A16 form of GPU
 * Kernel Lab, "Quantization experiments"; deq 2).  Only the n_ff products
 * are written.  g_p and u_p are reduced as gemv_q8_0 reduces an unsplit
 * row in that activation format.  Acceptance: the two GEMV bounds (of the
 * format) propagated through silu(g) u (slope of silu <= 1.1) plus 2^-20
 * relative for the fp32 epilogue.  n_ff >= 1, k % 32 == 0,
 * 32 <= k <= WSG_MAX_K_Q8ACT (WSG_MAX_K_F32ACT for f32) (WSG_ERR_SHAPE). */
int gemv_q8_0_swiglu(const void* w_packed, int64_t n_ff, int64_t k, const void* x, int act_fmt, float* y,
                     hipStream_t stream);

/* ------------------------------------------------ closing the decode loop
 * (GPU Kernel Lab, "Decode integration": fixed token/position buffers and
 * the LM-head GEMV + argmax + token/position update under one graph replay;
 * emit_qwen38_generate, "Where the speed comes from", item 2: token and
 * position advanced on the device, no host round trip per replay.)
 *
 * embed_gather: out[i] = row *token of the embedding table, as f32, i <
 *   hidden.  table: w_type WSG_W_Q8_0 (device layout, vocab rows, hidden %
 *   32 == 0; d * q is exact in f32) or WSG_W_BF16 (row-major vocab x hidden).
 *   token is read on the device when the kernel runs (e.g. the idx_out of
 *   lm_head_argmax); a token outside [0, vocab) gives a zero row.  Errors:
 *   vocab or hidden < 1 (WSG_ERR_SHAPE), bad w_type (WSG_ERR_MODE), null
 *   pointers, table not 16-byte or token/out not 4-byte aligned.
 * token_advance: history[*pos] = *token if 0 <= *pos < capacity, then
 *   *pos += 1 (one thread; the position keeps counting past capacity). */
int embed_gather(const void* table, int w_type, int64_t vocab, int64_t hidden, const int32_t* token, float* out,
                 hipStream_t stream);
int token_advance(const int32_t* token, int32_t* history, int64_t capacity, int32_t* pos, hipStream_t stream);

/* ------------------------------------------------------------- GEMVs ---
 * y[r] = sum_i W[r,i] x[i], f32 accumulation, r < n.  n == 0 is a no-op;
 * k == 0 writes y = 0.
 *
 * gemv_bf16: W row-major bf16 [n][k], k % 8 == 0, k <= WSG_MAX_K_F32ACT;
 *   x f32[k].  Acceptance: |y - y_ref| <= 2^-10 sum_i |w_i x_i| per row.
 * gemv_q8_0: W in the device layout; k % 32 == 0.  act_fmt as above.
 *   debug_block_dots (nullable; WSG_ACT_Q8_0 / _F32_REQUANT only) receives
 *   the exact int32 block dot products s[r][b] = sum_i qw[r,32b+i] qx[32b+i]
 *   as int32[n][k/32].  Acceptance: |y - y_ref| <= 1e-4 sum_b |d_w d_x s_b|
 *   (int8 paths), <= 1e-4 sum_b sum_i |d_w q_i x_i| (f32 path). */
int gemv_bf16(const uint16_t* w, int64_t n, int64_t k, const float* x, float* y, hipStream_t stream);
int gemv_q8_0(const void* w_packed, int64_t n, int64_t k, const void* x, int act_fmt, float* y,
              int32_t* debug_block_dots, hipStream_t stream);

/* Launch configuration a gemv_bf16 / gemv_q8_0 call of this shape would use
 * on the current device: waves per workgroup, waves that share one row
 * (split-K factor), chunks loaded ahead per wave (unroll), workgroups in the
 * grid and dynamic LDS bytes (outputs nullable).  For tooling; launches
 * nothing. */
int wsg_gemv_config(int w_type, int act_fmt, int64_t n, int64_t k, int* waves, int* split, int* unroll,
                    int* grid, int64_t* lds_bytes);

/* Tuning knobs for measurement sweeps (process-wide; 0 restores the
 * automatic choice).  WSG_TUNE_SPLITK: waves that share one row (1, 2 or
 * 4).  WSG_TUNE_WG_PER_CU: cap on workgroups per CU in the persistent grid.
 * WSG_TUNE_WAVES: waves per workgroup (4, 8 or 16).  WSG_TUNE_UNROLL:
 * 2048-weight chunks per weight item (1: three items in each wave's ring;
 * 2 or 4: two items; the requantizing path at most 2, the f32 path always
 * 1).  The debug and argmax variants keep the default (1).  Calls already
 * captured into a plan keep the configuration they were captured with.
 * Returns WSG_ERR_MODE for an unknown knob, WSG_ERR_SHAPE for a bad
 * value. */
enum { WSG_TUNE_SPLITK = 0, WSG_TUNE_WG_PER_CU = 1, WSG_TUNE_WAVES = 2, WSG_TUNE_UNROLL = 3 };
int wsg_tune(int knob, int value);

/* ------------------------------------------------- LM head + argmax ---
 * The LM-head GEMV (as gemv_bf16 / gemv_q8_0, w_type selects) fused with
 * stage 1 of a two-stage argmax: each workgroup reduces its rows' logits
 * to one key (value, lowest index among IEEE-equal values, -0 == +0) in
 * `ws`; stage 2 (one workgroup) writes the winning row index to *idx_out
 * in device memory.  The library never reads it back.  debug_logits
 * (nullable) receives the f32 logits.  n >= 1.  ws (8-byte aligned) must
 * hold 8 bytes per stage-1 workgroup: lm_head_argmax_ws_bytes(n, k, w_type)
 * bytes on the current device (any activation format), at most
 * wsg_argmax_ws_bytes() = 64 KiB for every shape (WSG_ERR_WORKSPACE if
 * smaller).  lm_head_argmax_ws_bytes returns -1 for a bad shape or type. */
int64_t wsg_argmax_ws_bytes(void);
int64_t lm_head_argmax_ws_bytes(int64_t n, int64_t k, int w_type);
int lm_head_argmax(const void* w, int w_type, int64_t n, int64_t k, const void* x, int act_fmt,
                   void* ws, size_t ws_bytes, int32_t* idx_out, float* debug_logits,
                   hipStream_t stream);

/* lm_head_argmax for callers that cannot allocate device memory (code
 * under hipGraph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, results and errors as lm_head_argmax,
 * but the stage-1 keys go to an array in the library's static device memory
 * instead of a caller workspace, so the call allocates nothing (no
 * hipMalloc or allocating library routine).  The array holds 8192 keys
 * (64 KiB) on every GPU the library runs on, until the process ends; a
 * shape whose stage 1 would need more keys gets WSG_ERR_WORKSPACE (no shape
 * that passes the other checks does).  Every call on one GPU uses that
 * GPU's array, which keeps the last call's keys; each call writes every key
 * it reads, so nothing needs clearing, but calls that overlap in time on
 * one GPU (two streams, two threads) race and give undefined indices.  The
 * first call on each device looks up the array's address (do it outside
 * stream capture); later calls are capturable. */
int lm_head_argmax_static(const void* w, int w_type, int64_t n, int64_t k, const void* x, int act_fmt,
                          int32_t* idx_out, float* debug_logits, hipStream_t stream);

/* The same two-stage argmax over an f32 vector v[n], n >= 1 (NaN outside
 * the contract); ws as above, at least wsg_argmax_ws_bytes() bytes. */
int argmax_f32(const float* v, int64_t n, void* ws, size_t ws_bytes, int32_t* idx_out,
               hipStream_t stream);

/* ------------------------------------------------- whole-token plan ---
 * A sequence of the calls above, captured once into a hipGraph and
 * replayed with one launch per token (emit_qwen38_generate, "Where the
 * speed comes from", item 2; qwen3-8b-rtx4080-cutedsl, "CUDA graphs").
 * Buffers are fixed at capture time: the caller keeps every buffer alive,
 * at the same address, until wsg_plan_destroy.  Replays reproduce the eager
 * results bit for bit. */
enum {
    WSG_OP_GEMV_BF16 = 0,       /* w, n, k, x (f32), y */
    WSG_OP_GEMV_Q8_0 = 1,       /* w, n, k, x, act_fmt, y */
    WSG_OP_QUANTIZE_ACT = 2,    /* x (f32), k, y = x_q8 output (void*) */
    WSG_OP_LM_HEAD_ARGMAX = 3,  /* w, w_type, n, k, x, act_fmt, ws, ws_bytes, idx_out */
    WSG_OP_RESIDUAL_RMSNORM = 4, /* residual_rmsnorm_q8_0: x = h, r, w = g, k, eps,
                                    h_out, y (f32 y), y_q8 */
    WSG_OP_GEMV_Q8_0_RMSNORM = 5, /* gemv_q8_0_rmsnorm (act_fmt WSG_ACT_F32: gemv_q8_0_rmsnorm_f32):
                                     w, n, k, x = h, r, g, eps, h_out, y */
    WSG_OP_GEMV_Q8_0_SWIGLU = 6,  /* gemv_q8_0_swiglu: w, n = n_ff, k, x, act_fmt, y */
    WSG_OP_EMBED_GATHER = 7,      /* embed_gather: w = table, w_type, n = vocab, k = hidden, x = token, y */
    WSG_OP_TOKEN_ADVANCE = 8,     /* token_advance: x = token, idx_out = history, n = capacity, ws = pos */
    WSG_OP_GEMV_Q4_0 = 9,         /* gemv_q4_0: w, n, k, x, act_fmt, y */
    WSG_OP_GEMV_Q4_0_RMSNORM = 10, /* gemv_q4_0_rmsnorm: w, n, k, x = h, r, g, eps, h_out, y */
    WSG_OP_GEMV_Q4_0_SWIGLU = 11, /* gemv_q4_0_swiglu: w, n = n_ff, k, x, act_fmt, y */
};

/* flags: WSG_OP_AFTER_ALL marks an op that depends on every earlier op of
 * the plan even where no buffer shows it (in a model, a layer's input is
 * computed from the previous layer's output by operators outside the plan).
 * Stream order already serializes the graph plan; the persistent plan makes
 * such an op wait until the previous op's whole output is written. */
enum { WSG_OP_AFTER_ALL = 1 };

typedef struct {
    int op;
    int w_type;
    int act_fmt;
    int64_t n;
    int64_t k;
    const void* w;
    const void* x;
    void* y;
    void* ws;
    size_t ws_bytes;
    int32_t* idx_out;
    int flags;
    /* WSG_OP_RESIDUAL_RMSNORM and the fused-norm GEMVs only (zero for every
     * other op) */
    const void* r;
    void* h_out;
    void* y_q8;
    float eps;
    const void* g; /* the fused-norm GEMVs' norm weight */
} wsg_op_desc;

typedef struct wsg_plan wsg_plan;

/* Validates every descriptor (first failure's status is returned, nothing
 * captured), then captures them in order.  `stream` is used for capture
 * only; it must not be capturing already. */
int wsg_plan_create(const wsg_op_desc* ops, int n_ops, hipStream_t stream, wsg_plan** out);
int wsg_plan_launch(wsg_plan* plan, hipStream_t stream);

/* Persistent whole-token plan: the same descriptors (Q8_0 GEMVs only, all
 * with WSG_ACT_F32_REQUANT or all with WSG_ACT_F32; f32 inputs) executed by
 * ONE kernel launch per replay, captured as a one-node hipGraph, with one
 * 16-wave workgroup per CU resident for the whole token.  Ops are ordered by
 * their data, not by grid barriers: an op whose x is (a slice of) an earlier
 * op's y reads each element as soon as its row is written, and a workgroup
 * requests the next matrix's first weights before it waits for that input,
 * so the weight stream does not drain between GEMVs.  Hence the plan
 * requires that each op's x is either wholly inside one earlier op's y or
 * overlaps no op's y at all, and that no y overlaps another op's y or an
 * input read from outside the plan (WSG_ERR_MODE otherwise).  Each op
 * reduces its rows in the same order as the eager call, so results equal
 * the eager calls' bit for bit.  An op may have at most 64 row tiles per
 * workgroup (rows <= 64 x CUs x 16 / split; 262,144 unsplit rows on 256
 * CUs), else WSG_ERR_SHAPE.
 * Unlike the hot calls, creating this plan allocates device memory (the
 * descriptor table, a launch counter, an error flag and two copies of every
 * op's output, one per launch parity) and synchronizes the device; do not
 * call it while a stream is capturing.  A wait that exceeds its spin limit
 * (about a second) makes the kernel give up rather than hang, every other
 * wait of that launch stops soon after, and wsg_plan_error reports it; the
 * plan's results are then invalid and it must be destroyed.  Replays of one
 * plan must not overlap in time (launch them on one stream). */
int wsg_plan_create_persistent(const wsg_op_desc* ops, int n_ops, hipStream_t stream, wsg_plan** out);

/* *flag = 1 if a persistent plan's wait ever timed out (its outputs are
 * then invalid), else 0.  Synchronizes the device (not capturable). */
int wsg_plan_error(wsg_plan* plan, int* flag);
/* Where the first wait that gave up was (all zero if none; synchronizes the
 * device): words[0] site (1: an input or dependency of an op not written
 * in time), words[1] workgroup, words[2] wave, words[3..5] zero. */
int wsg_plan_error_detail(wsg_plan* plan, int32_t* words);
int wsg_plan_destroy(wsg_plan* plan);
/* Number of kernel launches one replay makes. */
int wsg_plan_kernel_count(const wsg_plan* plan);
/* Shape of the persistent plan's kernel: waves per workgroup, 2048-weight
 * chunks per weight item and items in flight per wave (outputs nullable).
 * For tooling; launches nothing. */
int wsg_stream_config(int* waves, int* unroll, int* sets);

/* --------------------------------------------------- measurement tools ---
 * wsg_read_probe: reads `bytes` (multiple of 16) from buf with the same
 * load width and cache policy as the GEMV weight stream (each wave one
 * contiguous span, eight 1 KB wave loads in flight) and writes one float
 * per 256-thread workgroup to sink[blocks] so the reads are not elided;
 * blocks <= 0 picks four workgroups per CU.  wsg_copy_probe: dst[i] = src[i] for
 * `bytes` (multiple of 16): a kernel of exactly known traffic for
 * calibrating hardware byte counters. */
int wsg_read_probe(const void* buf, int64_t bytes, float* sink, int blocks, hipStream_t stream);
int wsg_copy_probe(const void* src, void* dst, int64_t bytes, hipStream_t stream);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif
#endif /* WSGEMV_H */
