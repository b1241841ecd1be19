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
#include "stream.hpp"
#include "wsgemv.h"

namespace wsg {
int validate_gemv_q8(const void* w, int64_t n, int64_t k, const void* x, int act_fmt, const void* y);
int validate_gemv_bf16(const void* w, int64_t n, int64_t k, const void* x, const void* y);
int validate_lm_head(const void* w, int w_type, int64_t n, int64_t k, const void* x, int act_fmt, const void* ws,
                     size_t ws_bytes, const void* idx_out);
int validate_residual_rmsnorm(const float* h, const float* r, const float* g, int64_t k, float eps,
                              const void* h_out, const void* y, const void* y_q8);
int validate_gemv_q8_rmsnorm(const void* w, int64_t n, int64_t k, const float* h, const float* r, const float* g,
                             float eps, const void* h_out, const void* y, int act_fmt);
int validate_gemv_q8_swiglu(const void* w, int64_t n_ff, int64_t k, const void* x, int act_fmt, const void* y);
int validate_embed_gather(const void* table, int w_type, int64_t vocab, int64_t hidden, const int32_t* token,
                          const float* out);
int validate_token_advance(const int32_t* token, const int32_t* history, int64_t capacity, const int32_t* pos);
int validate_gemv_q4(const void* w, int64_t n, int64_t k, const void* x, int act_fmt, const void* y);
int validate_gemv_q4_swiglu(const void* w, int64_t n_ff, int64_t k, const void* x, int act_fmt, const void* y);
}  // namespace wsg

struct wsg_plan {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int kernels = 0;
    // persistent plans: device descriptor table and barrier state
    void* ops_dev = nullptr;
    uint32_t* bar_dev = nullptr;
    void* tags_dev = nullptr;  // output copies of every op (two per op, by launch parity)
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
        case WSG_OP_RESIDUAL_RMSNORM:
            return wsg::validate_residual_rmsnorm(static_cast<const float*>(d.x), static_cast<const float*>(d.r),
                                                  static_cast<const float*>(d.w), d.k, d.eps, d.h_out, d.y,
                                                  d.y_q8);
        case WSG_OP_GEMV_Q8_0_RMSNORM:
            // act_fmt WSG_ACT_F32 selects the dequantizing (deq 2) form
            return wsg::validate_gemv_q8_rmsnorm(d.w, d.n, d.k, static_cast<const float*>(d.x),
                                                 static_cast<const float*>(d.r), static_cast<const float*>(d.g),
                                                 d.eps, d.h_out, d.y,
                                                 d.act_fmt == WSG_ACT_F32 ? WSG_ACT_F32 : WSG_ACT_F32_REQUANT);
        case WSG_OP_GEMV_Q8_0_SWIGLU: return wsg::validate_gemv_q8_swiglu(d.w, d.n, d.k, d.x, d.act_fmt, d.y);
        case WSG_OP_EMBED_GATHER:
            return wsg::validate_embed_gather(d.w, d.w_type, d.n, d.k, static_cast<const int32_t*>(d.x),
                                              static_cast<const float*>(d.y));
        case WSG_OP_TOKEN_ADVANCE:
            return wsg::validate_token_advance(static_cast<const int32_t*>(d.x), d.idx_out, d.n,
                                               static_cast<const int32_t*>(d.ws));
        case WSG_OP_GEMV_Q4_0: return wsg::validate_gemv_q4(d.w, d.n, d.k, d.x, d.act_fmt, d.y);
        case WSG_OP_GEMV_Q4_0_SWIGLU: return wsg::validate_gemv_q4_swiglu(d.w, d.n, d.k, d.x, d.act_fmt, d.y);
        case WSG_OP_GEMV_Q4_0_RMSNORM:
            return wsg::validate_gemv_q8_rmsnorm(d.w, d.n, d.k, static_cast<const float*>(d.x),
                                                 static_cast<const float*>(d.r), static_cast<const float*>(d.g),
                                                 d.eps, d.h_out, d.y, WSG_ACT_F32_REQUANT);
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
        case WSG_OP_RESIDUAL_RMSNORM:
            return residual_rmsnorm_q8_0(static_cast<const float*>(d.x), static_cast<const float*>(d.r),
                                         static_cast<const float*>(d.w), d.k, d.eps, static_cast<float*>(d.h_out),
                                         static_cast<float*>(d.y), d.y_q8, s);
        case WSG_OP_GEMV_Q8_0_RMSNORM:
            return (d.act_fmt == WSG_ACT_F32 ? gemv_q8_0_rmsnorm_f32 : gemv_q8_0_rmsnorm)(
                d.w, d.n, d.k, static_cast<const float*>(d.x), static_cast<const float*>(d.r),
                static_cast<const float*>(d.g), d.eps, static_cast<float*>(d.h_out), static_cast<float*>(d.y), s);
        case WSG_OP_GEMV_Q8_0_SWIGLU:
            return gemv_q8_0_swiglu(d.w, d.n, d.k, d.x, d.act_fmt, static_cast<float*>(d.y), s);
        case WSG_OP_EMBED_GATHER:
            return embed_gather(d.w, d.w_type, d.n, d.k, static_cast<const int32_t*>(d.x), static_cast<float*>(d.y),
                                s);
        case WSG_OP_TOKEN_ADVANCE:
            return token_advance(static_cast<const int32_t*>(d.x), d.idx_out, d.n, static_cast<int32_t*>(d.ws), s);
        case WSG_OP_GEMV_Q4_0: return gemv_q4_0(d.w, d.n, d.k, d.x, d.act_fmt, static_cast<float*>(d.y), s);
        case WSG_OP_GEMV_Q4_0_SWIGLU:
            return gemv_q4_0_swiglu(d.w, d.n, d.k, d.x, d.act_fmt, static_cast<float*>(d.y), s);
        case WSG_OP_GEMV_Q4_0_RMSNORM:
            return gemv_q4_0_rmsnorm(d.w, d.n, d.k, static_cast<const float*>(d.x), static_cast<const float*>(d.r),
                                     static_cast<const float*>(d.g), d.eps, static_cast<float*>(d.h_out),
                                     static_cast<float*>(d.y), s);
        default: return WSG_ERR_MODE;
    }
}

// Capture `enqueue(cap_stream)` into an instantiated graph held by `p`.
template <typename F>
int capture_into(wsg_plan* p, hipStream_t stream, F&& enqueue) {
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
    const int rc = enqueue(cap);
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
    p->graph = graph;
    p->exec = exec;
    p->kernels = kernels;
    return WSG_OK;
}

struct Range {
    uintptr_t lo, hi;
    bool overlaps(const Range& o) const { return lo < o.hi && o.lo < hi; }
};

void release(wsg_plan* p) {
    if (p->exec) (void)hipGraphExecDestroy(p->exec);
    if (p->graph) (void)hipGraphDestroy(p->graph);
    if (p->ops_dev) (void)hipFree(p->ops_dev);
    if (p->bar_dev) (void)hipFree(p->bar_dev);
    if (p->tags_dev) (void)hipFree(p->tags_dev);
    delete p;
}

}  // namespace

namespace {

// One resident kernel per replay (the whole token in one launch).
int create_resident(const wsg_op_desc* ops, int n_ops, hipStream_t stream, wsg_plan** out) {
    if (!ops || !out) return WSG_ERR_NULL;
    *out = nullptr;
    if (n_ops <= 0 || n_ops > 65536) return WSG_ERR_SHAPE;
    std::vector<wsg::StreamOp> table(n_ops);
    std::vector<int> producer(n_ops, -1);   // op whose output this op's x is, or -1
    std::vector<size_t> yc_off(n_ops, 0);   // element offset of each op's output copies
    std::vector<size_t> yc_stride(n_ops, 0);
    size_t yc_elems = 0;
    int max_k = 0;
    const bool f32 = ops[0].act_fmt == WSG_ACT_F32;
    for (int i = 0; i < n_ops; ++i) {
        const wsg_op_desc& d = ops[i];
        if (d.op != WSG_OP_GEMV_Q8_0) return WSG_ERR_MODE;
        if (d.act_fmt != WSG_ACT_F32_REQUANT && d.act_fmt != WSG_ACT_F32) return WSG_ERR_MODE;
        if ((d.act_fmt == WSG_ACT_F32) != f32) return WSG_ERR_MODE;  // one activation format per plan
        int rc = wsg::validate_gemv_q8(d.w, d.n, d.k, d.x, d.act_fmt, d.y);
        if (rc != WSG_OK) return rc;
        if (d.n < 1 || d.k < 32 || d.n > wsg::kMaxDim) return WSG_ERR_SHAPE;
        const Range rx{reinterpret_cast<uintptr_t>(d.x), reinterpret_cast<uintptr_t>(d.x) + 4 * (uintptr_t)d.k};
        const Range ry{reinterpret_cast<uintptr_t>(d.y), reinterpret_cast<uintptr_t>(d.y) + 4 * (uintptr_t)d.n};
        // Without grid barriers, ops run concurrently with every op that is
        // not an ancestor, so: the input is either wholly one earlier op's
        // output (read from its tagged copy, in dataflow order) or untouched
        // by any output of the plan; and no output may overlap another
        // output or any input read from outside the plan.
        for (int p = i - 1; p >= 0 && producer[i] < 0; --p) {
            const Range yp{reinterpret_cast<uintptr_t>(ops[p].y),
                           reinterpret_cast<uintptr_t>(ops[p].y) + 4 * (uintptr_t)ops[p].n};
            if (!yp.overlaps(rx)) continue;
            if (rx.lo < yp.lo || rx.hi > yp.hi || (rx.lo - yp.lo) % 4) return WSG_ERR_MODE;
            producer[i] = p;
        }
        for (int p = 0; p < n_ops; ++p) {
            const Range yp{reinterpret_cast<uintptr_t>(ops[p].y),
                           reinterpret_cast<uintptr_t>(ops[p].y) + 4 * (uintptr_t)ops[p].n};
            if (p != i && yp.overlaps(ry)) return WSG_ERR_MODE;
            if (producer[i] < 0 && yp.overlaps(rx) && p >= i) return WSG_ERR_MODE;
        }
        yc_off[i] = yc_elems;
        yc_stride[i] = ((size_t)d.n + 63) & ~(size_t)63;  // 256-byte aligned copies
        yc_elems += 2 * yc_stride[i];
        if (d.k > max_k) max_k = (int)d.k;
    }
    int waves = 0, grid = 0;
    size_t lds = 0;
    int rc = wsg::stream_config(max_k, f32, &waves, &grid, &lds);
    if (rc != WSG_OK) return rc;
    if ((int64_t)lds > wsg::device_info().max_lds) return WSG_ERR_SHAPE;
    for (int i = 0; i < n_ops; ++i)
        if (ops[i].n > wsg::stream_max_rows(wsg::stream_split(f32, ops[i].n, ops[i].k), grid)) return WSG_ERR_SHAPE;

    const size_t state_bytes = wsg::stream_state_bytes();
    wsg_plan* p = new (std::nothrow) wsg_plan;
    if (!p) return WSG_ERR_HIP;
    if (hipMalloc(&p->ops_dev, sizeof(wsg::StreamOp) * n_ops) != hipSuccess ||
        hipMalloc(reinterpret_cast<void**>(&p->bar_dev), state_bytes) != hipSuccess ||
        hipMalloc(&p->tags_dev, yc_elems * sizeof(float)) != hipSuccess) {
        release(p);
        return WSG_ERR_HIP;
    }
    float* copies = static_cast<float*>(p->tags_dev);
    for (int i = 0; i < n_ops; ++i) {
        const wsg_op_desc& d = ops[i];
        wsg::StreamOp& t = table[i];
        t.w = static_cast<const uint8_t*>(d.w);
        t.x = static_cast<const float*>(d.x);
        t.xs = nullptr;
        t.xs_stride = 0;
        if (producer[i] >= 0) {
            const int q = producer[i];
            const size_t off = (reinterpret_cast<uintptr_t>(d.x) - reinterpret_cast<uintptr_t>(ops[q].y)) / 4;
            t.xs = copies + yc_off[q] + off;
            t.xs_stride = (int64_t)yc_stride[q];
        }
        t.y = static_cast<float*>(d.y);
        t.ys = copies + yc_off[i];
        t.ys_stride = (int64_t)yc_stride[i];
        // an op marked as depending on everything before it waits for the
        // previous op's whole output (a later reader of it would)
        const bool after_all = (d.flags & WSG_OP_AFTER_ALL) != 0 && i > 0;
        t.dep = after_all ? copies + yc_off[i - 1] : nullptr;
        t.dep_stride = after_all ? (int64_t)yc_stride[i - 1] : 0;
        t.dep_n = after_all ? (int32_t)ops[i - 1].n : 0;
        t.n = (int32_t)d.n;
        t.k = (int32_t)d.k;
        t.act = d.act_fmt;
        t.split = wsg::stream_split(f32, d.n, d.k);
        t.pad = 0;
    }
    // the state starts at zero, every output copy at "not written"
    if (hipMemcpy(p->ops_dev, table.data(), sizeof(wsg::StreamOp) * n_ops, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemset(p->bar_dev, 0, state_bytes) != hipSuccess ||
        hipMemsetD32(reinterpret_cast<hipDeviceptr_t>(p->tags_dev), (int)wsg::kStreamSentinel, yc_elems) !=
            hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
        release(p);
        return WSG_ERR_HIP;
    }
    // a wait of more than ~2^20 polls (about a second) is a failure
    const int spin_limit = 1 << 20;
    const wsg::StreamOp* ops_dev = static_cast<const wsg::StreamOp*>(p->ops_dev);
    rc = capture_into(p, stream, [&](hipStream_t s) {
        return wsg::stream_launch(ops_dev, n_ops, f32, p->bar_dev, grid, lds, spin_limit, s);
    });
    if (rc != WSG_OK) {
        release(p);
        return rc;
    }
    *out = p;
    return WSG_OK;
}

}  // namespace

extern "C" {

int wsg_plan_create_persistent(const wsg_op_desc* ops, int n_ops, hipStream_t stream, wsg_plan** out) {
    return create_resident(ops, n_ops, stream, out);
}

int wsg_plan_error(wsg_plan* plan, int* flag) {
    if (!plan || !flag) return WSG_ERR_NULL;
    *flag = 0;
    if (!plan->bar_dev) return WSG_OK;
    uint32_t word = 0;
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&word, plan->bar_dev + wsg::stream_error_word(), sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
        return WSG_ERR_HIP;
    *flag = word != 0 ? 1 : 0;
    return WSG_OK;
}

int wsg_plan_error_detail(wsg_plan* plan, int32_t* words) {
    if (!plan || !words) return WSG_ERR_NULL;
    for (int i = 0; i < 6; ++i) words[i] = 0;
    if (!plan->bar_dev) return WSG_OK;
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(words, plan->bar_dev + wsg::stream_detail_word(), 6 * sizeof(int32_t), hipMemcpyDeviceToHost) !=
            hipSuccess)
        return WSG_ERR_HIP;
    return WSG_OK;
}

int wsg_plan_create(const wsg_op_desc* ops, int n_ops, hipStream_t stream, wsg_plan** out) {
    if (!ops || !out) return WSG_ERR_NULL;
    *out = nullptr;
    if (n_ops <= 0) return WSG_ERR_SHAPE;
    for (int i = 0; i < n_ops; ++i) {
        const int rc = validate_op(ops[i]);
        if (rc != WSG_OK) return rc;
    }
    (void)wsg::device_info();  // per-device lookups happen before capture
    wsg_plan* p = new (std::nothrow) wsg_plan;
    if (!p) return WSG_ERR_HIP;
    const int rc = capture_into(p, stream, [&](hipStream_t s) {
        int r = WSG_OK;
        for (int i = 0; i < n_ops && r == WSG_OK; ++i) r = enqueue_op(ops[i], s);
        return r;
    });
    if (rc != WSG_OK) {
        release(p);
        return rc;
    }
    *out = p;
    return WSG_OK;
}

int wsg_plan_launch(wsg_plan* plan, hipStream_t stream) {
    if (!plan || !plan->exec) return WSG_ERR_NULL;
    return hipGraphLaunch(plan->exec, stream) == hipSuccess ? WSG_OK : WSG_ERR_HIP;
}

int wsg_plan_destroy(wsg_plan* plan) {
    if (!plan) return WSG_ERR_NULL;
    release(plan);
    return WSG_OK;
}

int wsg_plan_kernel_count(const wsg_plan* plan) { return plan ? plan->kernels : -1; }

int wsg_stream_config(int* waves, int* unroll, int* sets) {
    int w = 0, u = 0, n = 0;
    wsg::stream_shape(&w, &u, &n);
    if (waves) *waves = w;
    if (unroll) *unroll = u;
    if (sets) *sets = n;
    return WSG_OK;
}

}  // extern "C"
