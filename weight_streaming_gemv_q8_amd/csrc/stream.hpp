// Descriptor of one GEMV of the persistent whole-token kernel, and the
// host-side hooks the plan uses to size and launch it.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wsg {

struct StreamOp {
    const uint8_t* w;       // Q8_0 weights, device layout
    const float* x;         // f32 input from outside the plan (xs == nullptr)
    const float* xs;        // or: the producer's output copy (parity 0) at x's offset
    float* y;               // f32 output
    float* ys;              // this op's output copies (parity 0; parity 1 at ys + ys_stride)
    const float* dep;       // output copy (parity 0) that must be complete first, or nullptr
    int64_t xs_stride, ys_stride, dep_stride;  // floats from a parity-0 copy to its parity-1 copy
    int32_t n, k;
    int32_t act;            // WSG_ACT_F32_REQUANT or WSG_ACT_F32
    int32_t split;          // waves per row: 1, 2 or 4
    int32_t dep_n;          // elements of dep
    int32_t pad;
};

// Bit pattern of a not-yet-written element of an output copy.
constexpr uint32_t kStreamSentinel = 0x7FA5A5A5u;

// Bytes of the state a plan allocates (zeroed once), and the index of its
// error word (uint32).
size_t stream_state_bytes();
size_t stream_error_word();
// First of the six words describing the first wait that gave up: site
// (1 input/dependency), workgroup, wave, op, expected value, value seen.
size_t stream_detail_word();

// Launch geometry of the persistent kernel for a chain whose largest k is
// max_k (f32: the ops keep f32 activations, else they requantize them).
int stream_config(int max_k, bool f32, int* waves, int* grid, size_t* lds);
int stream_launch(const StreamOp* ops_dev, int n_ops, bool f32, uint32_t* state_dev, int grid, size_t lds,
                  int spin_limit, hipStream_t stream);
int stream_split(bool f32, int64_t n, int64_t k);
// Waves per workgroup, chunks per ring item and ring items per wave.
void stream_shape(int* waves, int* unroll, int* sets);
// Most rows one op may have at a split factor and grid (the tiles of a
// workgroup wait in LDS until the op's end).
int64_t stream_max_rows(int split, int grid);

}  // namespace wsg
