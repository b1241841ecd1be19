// Descriptor of one GEMV of the persistent whole-token kernel, and the
// host-side hooks the plan uses to size and launch it.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wsg {

struct StreamOp {
    const uint8_t* w;  // Q8_0 weights, device layout
    const float* x;    // f32 input (quantized in the prologue unless act is f32)
    float* y;          // f32 output
    int32_t n, k;
    int32_t act;      // WSG_ACT_F32_REQUANT or WSG_ACT_F32
    int32_t split;    // waves per row: 1, 2 or 4
    int32_t barrier;  // 1: wait for every earlier op before reading x
    int32_t pad;
};

// Launch geometry of the persistent kernel for a chain whose largest k is
// max_k (f32: the ops keep f32 activations, else they requantize them).
int stream_config(int max_k, bool f32, int* waves, int* grid, size_t* lds);
int stream_launch(const StreamOp* ops_dev, int n_ops, bool f32, uint32_t* bar_dev, int grid, size_t lds,
                  int spin_limit, hipStream_t stream);
int stream_split(bool f32, int64_t n, int64_t k);

}  // namespace wsg
