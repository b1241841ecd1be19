"""Python binding of libwsgemv.so: batch-1 decode GEMV weight streaming on
MI355X (gfx950).

Argument marshalling only: every entry point forwards to the C ABI of the
same name (``include/wsgemv.h``), which does all of the work in HIP kernels.
Arguments that are device buffers may be torch tensors (their
``data_ptr()`` is passed) or raw integer addresses; ``stream`` defaults to
torch's current stream.  A nonzero status raises :class:`WsgError`.

The library must be built (``__graft_entry__.build()``); importing works
without it, but the first call raises if it is missing: there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwsgemv.so")

# status codes (wsgemv.h)
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_MODE, ERR_WORKSPACE, ERR_HIP = range(7)
# activation formats
ACT_Q8_0, ACT_F32, ACT_F32_REQUANT = 0, 1, 2
# weight types
W_BF16, W_Q8_0 = 0, 1
# plan ops
(OP_GEMV_BF16, OP_GEMV_Q8_0, OP_QUANTIZE_ACT, OP_LM_HEAD_ARGMAX, OP_RESIDUAL_RMSNORM, OP_GEMV_Q8_0_RMSNORM,
 OP_GEMV_Q8_0_SWIGLU, OP_EMBED_GATHER, OP_TOKEN_ADVANCE, OP_GEMV_Q4_0, OP_GEMV_Q4_0_RMSNORM,
 OP_GEMV_Q4_0_SWIGLU) = range(12)
OP_AFTER_ALL = 1  # OpDesc.flags: depends on every earlier op of the plan

MAX_K_Q8ACT = 57344
MAX_K_F32ACT = 36864

# exported C symbols, in header order
EXPORTS = (
    "wsg_status_str", "wsg_version", "q8_0_row_bytes", "q8_0_packed_bytes", "pack_q8_0",
    "quantize_q8_0_weights", "convert_bf16", "act_q8_0_bytes", "quantize_act_q8_0",
    "residual_rmsnorm_q8_0", "embed_gather", "token_advance", "q4_0_row_bytes", "q4_0_packed_bytes",
    "quantize_q4_0_weights", "gemv_q4_0", "gemv_q4_0_rmsnorm", "gemv_q4_0_swiglu", "gemv_q8_0_rmsnorm", "gemv_q8_0_rmsnorm_f32", "gemv_q8_0_swiglu",
    "gemv_bf16",
    "gemv_q8_0", "wsg_gemv_config", "wsg_tune", "wsg_argmax_ws_bytes", "lm_head_argmax_ws_bytes", "lm_head_argmax", "lm_head_argmax_static", "argmax_f32", "wsg_plan_create",
    "wsg_plan_launch", "wsg_plan_create_persistent", "wsg_plan_error", "wsg_plan_error_detail", "wsg_plan_destroy", "wsg_plan_kernel_count",
    "wsg_stream_config", "wsg_read_probe",
    "wsg_copy_probe",
)


class WsgError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_str(status)})")


class OpDesc(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int), ("w_type", ctypes.c_int), ("act_fmt", ctypes.c_int),
        ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("w", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t), ("idx_out", ctypes.c_void_p),
        ("flags", ctypes.c_int),
        ("r", ctypes.c_void_p), ("h_out", ctypes.c_void_p), ("y_q8", ctypes.c_void_p), ("eps", ctypes.c_float),
        ("g", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        # WSG_LIBRARY names another build of the same library (the diagnostic
        # timeline build, see timeline.py)
        path = os.environ.get("WSG_LIBRARY") or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(there is no fallback path)")
        L = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sig = {
            "wsg_status_str": (ctypes.c_char_p, [i32]),
            "wsg_version": (ctypes.c_char_p, []),
            "q8_0_row_bytes": (i64, [i64]),
            "q8_0_packed_bytes": (i64, [i64, i64]),
            "pack_q8_0": (i32, [vp, i64, i64, vp, vp]),
            "quantize_q8_0_weights": (i32, [vp, i64, i64, vp, vp]),
            "convert_bf16": (i32, [vp, i64, vp, vp]),
            "act_q8_0_bytes": (i64, [i64]),
            "quantize_act_q8_0": (i32, [vp, i64, vp, vp]),
            "residual_rmsnorm_q8_0": (i32, [vp, vp, vp, i64, ctypes.c_float, vp, vp, vp, vp]),
            "gemv_q8_0_rmsnorm": (i32, [vp, i64, i64, vp, vp, vp, ctypes.c_float, vp, vp, vp]),
            "gemv_q8_0_rmsnorm_f32": (i32, [vp, i64, i64, vp, vp, vp, ctypes.c_float, vp, vp, vp]),
            "gemv_q4_0_rmsnorm": (i32, [vp, i64, i64, vp, vp, vp, ctypes.c_float, vp, vp, vp]),
            "gemv_q8_0_swiglu": (i32, [vp, i64, i64, vp, i32, vp, vp]),
            "gemv_q4_0_swiglu": (i32, [vp, i64, i64, vp, i32, vp, vp]),
            "embed_gather": (i32, [vp, i32, i64, i64, vp, vp, vp]),
            "q4_0_row_bytes": (i64, [i64]),
            "q4_0_packed_bytes": (i64, [i64, i64]),
            "quantize_q4_0_weights": (i32, [vp, i64, i64, vp, vp]),
            "gemv_q4_0": (i32, [vp, i64, i64, vp, i32, vp, vp]),
            "token_advance": (i32, [vp, vp, i64, vp, vp]),
            "gemv_bf16": (i32, [vp, i64, i64, vp, vp, vp]),
            "gemv_q8_0": (i32, [vp, i64, i64, vp, i32, vp, vp, vp]),
            "wsg_gemv_config": (i32, [i32, i32, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                       ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i64)]),
            "wsg_tune": (i32, [i32, i32]),
            "wsg_argmax_ws_bytes": (i64, []),
            "lm_head_argmax_ws_bytes": (i64, [i64, i64, i32]),
            "lm_head_argmax": (i32, [vp, i32, i64, i64, vp, i32, vp, ctypes.c_size_t, vp, vp, vp]),
            "lm_head_argmax_static": (i32, [vp, i32, i64, i64, vp, i32, vp, vp, vp]),
            "argmax_f32": (i32, [vp, i64, vp, ctypes.c_size_t, vp, vp]),
            "wsg_plan_create": (i32, [ctypes.POINTER(OpDesc), i32, vp, ctypes.POINTER(vp)]),
            "wsg_plan_launch": (i32, [vp, vp]),
            "wsg_plan_create_persistent": (i32, [ctypes.POINTER(OpDesc), i32, vp, ctypes.POINTER(vp)]),
            "wsg_plan_error": (i32, [vp, ctypes.POINTER(i32)]),
            "wsg_plan_error_detail": (i32, [vp, ctypes.POINTER(i32)]),
            "wsg_plan_destroy": (i32, [vp]),
            "wsg_plan_kernel_count": (i32, [vp]),
            "wsg_stream_config": (i32, [ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]),
            "wsg_read_probe": (i32, [vp, i64, vp, i32, vp]),
            "wsg_copy_probe": (i32, [vp, vp, i64, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().wsg_status_str(status).decode()


def version() -> str:
    return lib().wsg_version().decode()


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise WsgError(fn, status)


# ---------------------------------------------------------------- sizes

def q8_0_row_bytes(k: int) -> int:
    return int(lib().q8_0_row_bytes(k))


def q8_0_packed_bytes(n: int, k: int) -> int:
    return int(lib().q8_0_packed_bytes(n, k))


def act_q8_0_bytes(k: int) -> int:
    return int(lib().act_q8_0_bytes(k))


def argmax_ws_bytes() -> int:
    return int(lib().wsg_argmax_ws_bytes())


def lm_head_argmax_ws_bytes(n: int, k: int, w_type: int) -> int:
    """Workspace the LM-head argmax of this shape needs on the current device."""
    v = int(lib().lm_head_argmax_ws_bytes(n, k, w_type))
    if v < 0:
        raise WsgError("lm_head_argmax_ws_bytes", ERR_SHAPE)
    return v


# --------------------------------------------------------- weight prep

def pack_q8_0(blocks_aos, n: int, k: int, w_packed, stream=None) -> None:
    _check("pack_q8_0", lib().pack_q8_0(_ptr(blocks_aos), n, k, _ptr(w_packed), _stream(stream)))


def quantize_q8_0_weights(w, n: int, k: int, w_packed, stream=None) -> None:
    _check("quantize_q8_0_weights",
           lib().quantize_q8_0_weights(_ptr(w), n, k, _ptr(w_packed), _stream(stream)))


def convert_bf16(src, count: int, out, stream=None) -> None:
    _check("convert_bf16", lib().convert_bf16(_ptr(src), count, _ptr(out), _stream(stream)))


def quantize_act_q8_0(x, k: int, x_q8, stream=None) -> None:
    _check("quantize_act_q8_0", lib().quantize_act_q8_0(_ptr(x), k, _ptr(x_q8), _stream(stream)))


def residual_rmsnorm_q8_0(h, r, g, k: int, eps: float, h_out=None, y=None, y_q8=None, stream=None) -> None:
    """h' = h + r, y = h' / sqrt(mean(h'^2) + eps) * g, y_q8 = Q8_0(y); r, g and
    each output may be None."""
    _check("residual_rmsnorm_q8_0",
           lib().residual_rmsnorm_q8_0(_ptr(h), _ptr(r), _ptr(g), k, eps, _ptr(h_out), _ptr(y), _ptr(y_q8),
                                       _stream(stream)))


def gemv_q8_0_rmsnorm(w_packed, n: int, k: int, h, r, g, eps: float, y, h_out=None, stream=None) -> None:
    """y = W . Q8_0(RMSNorm(h + r) * g), the norm computed in the GEMV's
    prologue; h + r goes to h_out (r, g and h_out may be None)."""
    _check("gemv_q8_0_rmsnorm",
           lib().gemv_q8_0_rmsnorm(_ptr(w_packed), n, k, _ptr(h), _ptr(r), _ptr(g), eps, _ptr(h_out), _ptr(y),
                                   _stream(stream)))


def gemv_q8_0_rmsnorm_f32(w_packed, n: int, k: int, h, r, g, eps: float, y, h_out=None, stream=None) -> None:
    """The deq 2 form: y = W . (RMSNorm(h + r) * g) with f32 activations, the
    norm computed in the GEMV's prologue."""
    _check("gemv_q8_0_rmsnorm_f32",
           lib().gemv_q8_0_rmsnorm_f32(_ptr(w_packed), n, k, _ptr(h), _ptr(r), _ptr(g), eps, _ptr(h_out), _ptr(y),
                                       _stream(stream)))


def gemv_q4_0_rmsnorm(w_packed, n: int, k: int, h, r, g, eps: float, y, h_out=None, stream=None) -> None:
    """The 4-bit form of gemv_q8_0_rmsnorm: y = W . Q8_0(RMSNorm(h + r) * g)
    with W in the 4-bit layout."""
    _check("gemv_q4_0_rmsnorm",
           lib().gemv_q4_0_rmsnorm(_ptr(w_packed), n, k, _ptr(h), _ptr(r), _ptr(g), eps, _ptr(h_out), _ptr(y),
                                   _stream(stream)))


def q4_0_row_bytes(k: int) -> int:
    return int(lib().q4_0_row_bytes(k))


def q4_0_packed_bytes(n: int, k: int) -> int:
    return int(lib().q4_0_packed_bytes(n, k))


def quantize_q4_0_weights(w, n: int, k: int, w_packed, stream=None) -> None:
    """f32 [n, k] -> 4-bit blocks in the device layout (see gemv_q4_0)."""
    _check("quantize_q4_0_weights", lib().quantize_q4_0_weights(_ptr(w), n, k, _ptr(w_packed), _stream(stream)))


def gemv_q4_0(w_packed, n: int, k: int, x, act_fmt: int, y, stream=None) -> None:
    """y = W x for 4-bit weights, int8 activations (ACT_Q8_0 or ACT_F32_REQUANT)."""
    _check("gemv_q4_0", lib().gemv_q4_0(_ptr(w_packed), n, k, _ptr(x), act_fmt, _ptr(y), _stream(stream)))


def embed_gather(table, w_type: int, vocab: int, hidden: int, token, out, stream=None) -> None:
    """out = row *token of the embedding table (read on the device), as f32."""
    _check("embed_gather", lib().embed_gather(_ptr(table), w_type, vocab, hidden, _ptr(token), _ptr(out),
                                              _stream(stream)))


def token_advance(token, history, capacity: int, pos, stream=None) -> None:
    """history[*pos] = *token (while *pos < capacity), *pos += 1, on the device."""
    _check("token_advance", lib().token_advance(_ptr(token), _ptr(history), capacity, _ptr(pos), _stream(stream)))


def gemv_q8_0_swiglu(w_packed, n_ff: int, k: int, x, act_fmt: int, y, stream=None) -> None:
    """y[p] = silu(W[p].x) * W[n_ff + p].x for the gate+up matrix (2 n_ff rows)."""
    _check("gemv_q8_0_swiglu", lib().gemv_q8_0_swiglu(_ptr(w_packed), n_ff, k, _ptr(x), act_fmt, _ptr(y),
                                                      _stream(stream)))


def gemv_q4_0_swiglu(w_packed, n_ff: int, k: int, x, act_fmt: int, y, stream=None) -> None:
    """gemv_q8_0_swiglu on a gate+up matrix in the 4-bit layout."""
    _check("gemv_q4_0_swiglu", lib().gemv_q4_0_swiglu(_ptr(w_packed), n_ff, k, _ptr(x), act_fmt, _ptr(y),
                                                      _stream(stream)))


# ------------------------------------------------------------------ GEMV

def gemv_bf16(w, n: int, k: int, x, y, stream=None) -> None:
    _check("gemv_bf16", lib().gemv_bf16(_ptr(w), n, k, _ptr(x), _ptr(y), _stream(stream)))


def gemv_q8_0(w_packed, n: int, k: int, x, act_fmt: int, y, debug_block_dots=None, stream=None) -> None:
    _check("gemv_q8_0", lib().gemv_q8_0(_ptr(w_packed), n, k, _ptr(x), act_fmt, _ptr(y),
                                        _ptr(debug_block_dots), _stream(stream)))


def gemv_config(w_type: int, act_fmt: int, n: int, k: int) -> dict:
    """Launch configuration the library uses for this call shape."""
    w, s, u, g = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    lds = ctypes.c_int64()
    _check("wsg_gemv_config", lib().wsg_gemv_config(w_type, act_fmt, n, k, ctypes.byref(w), ctypes.byref(s),
                                                    ctypes.byref(u), ctypes.byref(g), ctypes.byref(lds)))
    return {"waves": w.value, "split": s.value, "unroll": u.value, "grid": g.value, "lds_bytes": lds.value}


def stream_config() -> dict:
    """Shape of the persistent token kernel."""
    w, u, n = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check("wsg_stream_config", lib().wsg_stream_config(ctypes.byref(w), ctypes.byref(u), ctypes.byref(n)))
    return {"waves": w.value, "unroll": u.value, "sets": n.value}


TUNE_SPLITK, TUNE_WG_PER_CU, TUNE_WAVES, TUNE_UNROLL = 0, 1, 2, 3


def tune(knob: int, value: int) -> None:
    """Process-wide launch-configuration override for sweeps (0 = automatic)."""
    _check("wsg_tune", lib().wsg_tune(knob, value))


def lm_head_argmax(w, w_type: int, n: int, k: int, x, act_fmt: int, ws, ws_bytes: int, idx_out,
                   debug_logits=None, stream=None) -> None:
    _check("lm_head_argmax", lib().lm_head_argmax(_ptr(w), w_type, n, k, _ptr(x), act_fmt, _ptr(ws),
                                                  ws_bytes, _ptr(idx_out), _ptr(debug_logits),
                                                  _stream(stream)))


def lm_head_argmax_static(w, w_type: int, n: int, k: int, x, act_fmt: int, idx_out, debug_logits=None,
                          stream=None) -> None:
    """lm_head_argmax without a workspace (keys in the library's static array)."""
    _check("lm_head_argmax_static", lib().lm_head_argmax_static(_ptr(w), w_type, n, k, _ptr(x), act_fmt,
                                                                _ptr(idx_out), _ptr(debug_logits),
                                                                _stream(stream)))


def argmax_f32(v, n: int, ws, ws_bytes: int, idx_out, stream=None) -> None:
    _check("argmax_f32", lib().argmax_f32(_ptr(v), n, _ptr(ws), ws_bytes, _ptr(idx_out), _stream(stream)))


# ------------------------------------------------------------------ plan

def op_gemv_q8_0(w, n, k, x, act_fmt, y) -> OpDesc:
    return OpDesc(op=OP_GEMV_Q8_0, w_type=W_Q8_0, act_fmt=act_fmt, n=n, k=k, w=_ptr(w), x=_ptr(x), y=_ptr(y))


def op_gemv_q8_0_rmsnorm(w, n, k, h, r, g, eps, y, h_out=None, act_fmt=None) -> OpDesc:
    """act_fmt ACT_F32 selects the dequantizing form (gemv_q8_0_rmsnorm_f32)."""
    return OpDesc(op=OP_GEMV_Q8_0_RMSNORM, w_type=W_Q8_0, act_fmt=ACT_F32_REQUANT if act_fmt is None else act_fmt,
                  n=n, k=k, w=_ptr(w), x=_ptr(h), r=_ptr(r), g=_ptr(g), eps=eps, h_out=_ptr(h_out), y=_ptr(y))


def op_gemv_q8_0_swiglu(w, n_ff, k, x, act_fmt, y) -> OpDesc:
    return OpDesc(op=OP_GEMV_Q8_0_SWIGLU, w_type=W_Q8_0, act_fmt=act_fmt, n=n_ff, k=k, w=_ptr(w), x=_ptr(x),
                  y=_ptr(y))


def op_gemv_q4_0_swiglu(w, n_ff, k, x, act_fmt, y) -> OpDesc:
    return OpDesc(op=OP_GEMV_Q4_0_SWIGLU, act_fmt=act_fmt, n=n_ff, k=k, w=_ptr(w), x=_ptr(x), y=_ptr(y))


def op_gemv_q4_0(w, n, k, x, act_fmt, y) -> OpDesc:
    return OpDesc(op=OP_GEMV_Q4_0, act_fmt=act_fmt, n=n, k=k, w=_ptr(w), x=_ptr(x), y=_ptr(y))


def op_gemv_q4_0_rmsnorm(w, n, k, h, r, g, eps, y, h_out=None) -> OpDesc:
    return OpDesc(op=OP_GEMV_Q4_0_RMSNORM, act_fmt=ACT_F32_REQUANT, n=n, k=k, w=_ptr(w), x=_ptr(h), r=_ptr(r),
                  g=_ptr(g), eps=eps, h_out=_ptr(h_out), y=_ptr(y))


def op_embed_gather(table, w_type, vocab, hidden, token, out) -> OpDesc:
    return OpDesc(op=OP_EMBED_GATHER, w_type=w_type, n=vocab, k=hidden, w=_ptr(table), x=_ptr(token), y=_ptr(out))


def op_token_advance(token, history, capacity, pos) -> OpDesc:
    return OpDesc(op=OP_TOKEN_ADVANCE, n=capacity, x=_ptr(token), idx_out=_ptr(history), ws=_ptr(pos))


def op_gemv_bf16(w, n, k, x, y) -> OpDesc:
    return OpDesc(op=OP_GEMV_BF16, w_type=W_BF16, act_fmt=ACT_F32, n=n, k=k, w=_ptr(w), x=_ptr(x), y=_ptr(y))


def op_quantize_act(x, k, x_q8) -> OpDesc:
    return OpDesc(op=OP_QUANTIZE_ACT, k=k, x=_ptr(x), y=_ptr(x_q8))


def op_lm_head_argmax(w, w_type, n, k, x, act_fmt, ws, ws_bytes, idx_out, debug_logits=None) -> OpDesc:
    return OpDesc(op=OP_LM_HEAD_ARGMAX, w_type=w_type, act_fmt=act_fmt, n=n, k=k, w=_ptr(w), x=_ptr(x),
                  y=_ptr(debug_logits), ws=_ptr(ws), ws_bytes=ws_bytes, idx_out=_ptr(idx_out))


def op_residual_rmsnorm(h, r, g, k, eps, h_out=None, y=None, y_q8=None) -> OpDesc:
    return OpDesc(op=OP_RESIDUAL_RMSNORM, k=k, x=_ptr(h), r=_ptr(r), w=_ptr(g), eps=eps, h_out=_ptr(h_out),
                  y=_ptr(y), y_q8=_ptr(y_q8))


class Plan:
    """A captured whole-token sequence of calls (hipGraph), replayed by launch().
    persistent=True runs the whole sequence in one resident kernel launch."""

    def __init__(self, ops: Sequence[OpDesc], stream=None, persistent: bool = False):
        arr = (OpDesc * len(ops))(*ops)
        h = ctypes.c_void_p()
        fn = "wsg_plan_create_persistent" if persistent else "wsg_plan_create"
        _check(fn, getattr(lib(), fn)(arr, len(ops), _stream(stream), ctypes.byref(h)))
        self._h = h
        self.n_ops = len(ops)
        self.persistent = persistent

    def error(self) -> bool:
        """True if a persistent plan's wait timed out (outputs invalid); synchronizes."""
        f = ctypes.c_int()
        _check("wsg_plan_error", lib().wsg_plan_error(self._h, ctypes.byref(f)))
        return bool(f.value)

    def error_detail(self) -> dict:
        """Where the first wait that gave up was (site 0: none); synchronizes."""
        w = (ctypes.c_int32 * 6)()
        _check("wsg_plan_error_detail", lib().wsg_plan_error_detail(self._h, w))
        sites = {0: "none", 1: "input or dependency"}
        return {"site": sites.get(w[0], str(w[0])), "workgroup": w[1], "wave": w[2], "op": w[3],
                "awaited": w[4], "seen": w[5]}

    @property
    def kernel_count(self) -> int:
        return int(lib().wsg_plan_kernel_count(self._h))

    def launch(self, stream=None) -> None:
        _check("wsg_plan_launch", lib().wsg_plan_launch(self._h, _stream(stream)))

    def destroy(self) -> None:
        if self._h:
            _check("wsg_plan_destroy", lib().wsg_plan_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            if self._h:
                lib().wsg_plan_destroy(self._h)
        except Exception:
            pass


# ----------------------------------------------------------- measurement

def read_probe(buf, nbytes: int, sink, blocks: int = 0, stream=None) -> None:
    _check("wsg_read_probe", lib().wsg_read_probe(_ptr(buf), nbytes, _ptr(sink), blocks, _stream(stream)))


def copy_probe(src, dst, nbytes: int, stream=None) -> None:
    _check("wsg_copy_probe", lib().wsg_copy_probe(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


# deq modes of the LM head and layer GEMVs (emit_qwen38_generate: 0 = int8
# activations everywhere, 1 = f32 for the LM head only, 2 = f32 for every
# Q8_0 GEMV)
def act_fmt_for(deq: int, lm_head: bool, fused_requant: bool = True) -> int:
    if deq not in (0, 1, 2):
        raise ValueError("deq must be 0, 1 or 2")
    if deq == 2 or (deq == 1 and lm_head):
        return ACT_F32
    return ACT_F32_REQUANT if fused_requant else ACT_Q8_0
