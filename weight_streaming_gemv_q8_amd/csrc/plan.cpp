// Whole-token plan: a fixed sequence of GEMV / quantize / LM-head calls
// captured once into a hipGraph and replayed with one launch per token
// (emit_qwen38_generate, "Where the speed comes from", item 2: hundreds of
// kernels per token at a few microseconds of launch overhead each would
// cost milliseconds; qwen3-8b-rtx4080-cutedsl, "CUDA graphs": static shapes
// and pre-allocated buffers).  The graph holds kernel nodes only; no memset
// or copy nodes are recorded.
#include <hip/hip_runtime.h>

#include <new>
#include <vector>

#include "internal.hpp"
#include "wsgemv.h"

namespace wsg {
int validate_gemv_q8(const void* w, int64_t n, int64_t k, const void* x, int act_fmt, const void* y);
int validate_gemv_bf16(const void* w, int64_t n, int64_t k, const void* x, const void* y);
int validate_lm_head(const void* w, int w_type, int64_t n, int64_t k, const void* x, int act_fmt, const void* ws,
                     size_t ws_bytes, const void* idx_out);
}  // namespace wsg

struct wsg_plan {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int kernels = 0;
};

namespace {

int validate_op(const wsg_op_desc& d) {
    switch (d.op) {
        case WSG_OP_GEMV_BF16: return wsg::validate_gemv_bf16(d.w, d.n, d.k, d.x, d.y);
        case WSG_OP_GEMV_Q8_0: return wsg::validate_gemv_q8(d.w, d.n, d.k, d.x, d.act_fmt, d.y);
        case WSG_OP_QUANTIZE_ACT:
            if (d.k < 0 || d.k % 32) return WSG_ERR_SHAPE;
            if (d.k > 0 && (!d.x || !d.y)) return WSG_ERR_NULL;
            if (d.k > 0 && (!wsg::aligned(d.x, 16) || !wsg::aligned(d.y, 16))) return WSG_ERR_ALIGN;
            return WSG_OK;
        case WSG_OP_LM_HEAD_ARGMAX:
            return wsg::validate_lm_head(d.w, d.w_type, d.n, d.k, d.x, d.act_fmt, d.ws, d.ws_bytes, d.idx_out);
        default: return WSG_ERR_MODE;
    }
}

int enqueue_op(const wsg_op_desc& d, hipStream_t s) {
    switch (d.op) {
        case WSG_OP_GEMV_BF16:
            return gemv_bf16(static_cast<const uint16_t*>(d.w), d.n, d.k, static_cast<const float*>(d.x),
                             static_cast<float*>(d.y), s);
        case WSG_OP_GEMV_Q8_0:
            return gemv_q8_0(d.w, d.n, d.k, d.x, d.act_fmt, static_cast<float*>(d.y), nullptr, s);
        case WSG_OP_QUANTIZE_ACT: return quantize_act_q8_0(static_cast<const float*>(d.x), d.k, d.y, s);
        case WSG_OP_LM_HEAD_ARGMAX:
            return lm_head_argmax(d.w, d.w_type, d.n, d.k, d.x, d.act_fmt, d.ws, d.ws_bytes, d.idx_out,
                                  static_cast<float*>(d.y), s);
        default: return WSG_ERR_MODE;
    }
}

}  // namespace

extern "C" {

int wsg_plan_create(const wsg_op_desc* ops, int n_ops, hipStream_t stream, wsg_plan** out) {
    if (!ops || !out) return WSG_ERR_NULL;
    *out = nullptr;
    if (n_ops <= 0) return WSG_ERR_SHAPE;
    for (int i = 0; i < n_ops; ++i) {
        const int rc = validate_op(ops[i]);
        if (rc != WSG_OK) return rc;
    }
    (void)wsg::device_info();  // per-device lookups happen before capture

    hipStream_t cap = stream;
    bool own = false;
    if (cap == nullptr) {
        if (hipStreamCreateWithFlags(&cap, hipStreamNonBlocking) != hipSuccess) return WSG_ERR_HIP;
        own = true;
    }
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(cap, &st) != hipSuccess || st != hipStreamCaptureStatusNone) {
        if (own) (void)hipStreamDestroy(cap);
        return WSG_ERR_MODE;
    }
    if (hipStreamBeginCapture(cap, hipStreamCaptureModeRelaxed) != hipSuccess) {
        if (own) (void)hipStreamDestroy(cap);
        return WSG_ERR_HIP;
    }
    int rc = WSG_OK;
    for (int i = 0; i < n_ops && rc == WSG_OK; ++i) rc = enqueue_op(ops[i], cap);
    hipGraph_t graph = nullptr;
    const hipError_t end = hipStreamEndCapture(cap, &graph);
    if (own) (void)hipStreamDestroy(cap);
    if (rc != WSG_OK || end != hipSuccess || graph == nullptr) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc != WSG_OK ? rc : WSG_ERR_HIP;
    }
    hipGraphExec_t exec = nullptr;
    if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
        (void)hipGraphDestroy(graph);
        return WSG_ERR_HIP;
    }
    size_t count = 0;
    int kernels = 0;
    if (hipGraphGetNodes(graph, nullptr, &count) == hipSuccess && count > 0) {
        std::vector<hipGraphNode_t> nodes(count);
        if (hipGraphGetNodes(graph, nodes.data(), &count) == hipSuccess) {
            for (size_t i = 0; i < count; ++i) {
                hipGraphNodeType t;
                if (hipGraphNodeGetType(nodes[i], &t) == hipSuccess && t == hipGraphNodeTypeKernel) ++kernels;
            }
        }
    }
    wsg_plan* p = new (std::nothrow) wsg_plan;
    if (!p) {
        (void)hipGraphExecDestroy(exec);
        (void)hipGraphDestroy(graph);
        return WSG_ERR_HIP;
    }
    p->graph = graph;
    p->exec = exec;
    p->kernels = kernels;
    *out = p;
    return WSG_OK;
}

int wsg_plan_launch(wsg_plan* plan, hipStream_t stream) {
    if (!plan || !plan->exec) return WSG_ERR_NULL;
    return hipGraphLaunch(plan->exec, stream) == hipSuccess ? WSG_OK : WSG_ERR_HIP;
}

int wsg_plan_destroy(wsg_plan* plan) {
    if (!plan) return WSG_ERR_NULL;
    int rc = WSG_OK;
    if (plan->exec && hipGraphExecDestroy(plan->exec) != hipSuccess) rc = WSG_ERR_HIP;
    if (plan->graph && hipGraphDestroy(plan->graph) != hipSuccess) rc = WSG_ERR_HIP;
    delete plan;
    return rc;
}

int wsg_plan_kernel_count(const wsg_plan* plan) { return plan ? plan->kernels : -1; }

}  // extern "C"
