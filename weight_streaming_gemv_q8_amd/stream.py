"""A whole-token batch-1 GEMV chain held resident in HBM, and its captured
plan (emit_qwen38_generate, "Where the speed comes from": one launch per
concatenated projection, one graph per token).

Per layer the chain is ``len(shapes)`` GEMVs.  The first reads the layer's
own input vector; each later GEMV reads the first K entries of the previous
GEMV's output (the projections' data flow within a layer; the non-GEMV
operators between them are not part of this path).  Every GEMV writes its
own output buffer, so all intermediates stay readable after a replay.

With ``norm_before`` the chain also carries the residual stream between
the GEMVs (item 3 of the same section: the residual add, the next RMSNorm
and the activation re-quantization in one kernel): before each listed GEMV
a residual_rmsnorm_q8_0 call adds the previous GEMV's output (the previous
layer's last GEMV for a layer's first) to the residual stream and feeds the
GEMV the normalized, re-quantized result.  Each such call writes its own
buffers, so a replay is a pure function of the token's input vector and
the weights, and every intermediate stays readable.

Weights live in one allocation; concatenated projections are filled part by
part into consecutive row ranges.  How the weight values are produced is
left to the caller (``fill_q8`` / ``fill_bf16`` callbacks that write f32
rows into a device staging buffer); this module only lays the buffers out
and drives the library.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Sequence, Tuple

import torch

import weight_streaming_gemv_q8_amd as wsg

ALIGN = 256


def _align(v: int, a: int = ALIGN) -> int:
    return (v + a - 1) // a * a


@dataclass(eq=False)
class GemvSlot:
    layer: int
    index: int
    n: int
    k: int
    w_offset: int      # byte offset into the weight allocation
    w_bytes: int
    x_ptr: int = 0     # f32 input (layer input or previous output)
    xq_ptr: int = 0    # quantized-activation buffer (separate-requant mode only)
    y: torch.Tensor = None
    norm: "NormSlot" = None  # the residual + RMSNorm call feeding this GEMV


@dataclass(eq=False)
class NormSlot:
    layer: int
    index: int              # the GEMV it feeds
    h_in: int = 0           # residual stream before the add
    r: int = 0              # added output (0: none)
    g: int = 0              # gain vector
    h_out: torch.Tensor = None
    y: torch.Tensor = None  # f32 normalized vector
    yq: torch.Tensor = None  # its Q8_0 activation (int8 paths)


class TokenStream:
    """Buffers of one token's GEMV chain.

    shapes: per-layer list of (rows n, k, parts) with parts the row counts of
            the stacked projections.
    wtype:  "q8_0" or "bf16".
    deq:    0, 1 or 2 (the deq modes); deq 0/1 use int8 activations on every
            layer GEMV.  BF16 chains ignore it.
    requant: "fused" (the GEMV quantizes its f32 input itself) or
            "separate" (a quantize_act_q8_0 launch before each GEMV).
    norm_before: indices of the GEMVs of a layer that read the residual
            stream through a residual add + RMSNorm (e.g. (0, 2): the
            attention input and the MLP input); each such GEMV's k, and the
            rows of the GEMV before it, are the hidden size.  Empty: every
            layer starts from its own input vector (set_inputs).
    eps:    the RMSNorm epsilon.
    swiglu_at: indices of the GEMVs of a layer whose output is the SwiGLU
            of their two halves (the gate+up projection: rows 0 .. n/2 - 1
            are the gate, the rest the up projection; gemv_q8_0_swiglu),
            so the next GEMV reads n/2 products.  Q8_0 chains (the W8A16
            form at deq 2) and q4_0 chains with int8 activations.
    fused_norm: with norm_before on a Q8_0 chain or a q4_0 chain with int8
            activations, each normalized GEMV computes the residual add +
            RMSNorm itself (gemv_q8_0_rmsnorm, or gemv_q8_0_rmsnorm_f32 at
            deq 2) instead of after a separate norm call; the results are
            the same bit for bit (the f32 normalized vectors are then not
            written).  A normalized SwiGLU GEMV keeps its separate norm call.
    """

    def __init__(self, shapes: Sequence[Tuple[int, int, Tuple[int, ...]]], layers: int, wtype: str,
                 deq: int = 0, requant: str = "fused", device: str = "cuda",
                 norm_before: Sequence[int] = (), eps: float = 1e-6, fused_norm: bool = False,
                 swiglu_at: Sequence[int] = ()):
        if wtype not in ("q8_0", "q4_0", "bf16"):
            raise ValueError("wtype must be q8_0, q4_0 or bf16")
        if wtype == "q4_0" and (requant != "fused" or ((norm_before or swiglu_at) and deq == 2)):
            raise ValueError("q4_0 chains run f32 activations (deq 2) or int8 ones requantized in each GEMV "
                             "or by the norm step")
        if requant not in ("fused", "separate"):
            raise ValueError("requant must be fused or separate")
        self.shapes = [(int(n), int(k), tuple(p)) for n, k, p in shapes]
        self.layers = layers
        self.wtype = wtype
        self.deq = deq
        self.requant = requant
        self.device = device
        self.swiglu_at = tuple(sorted(set(int(j) for j in swiglu_at)))
        for j in self.swiglu_at:
            if not 0 <= j < len(self.shapes) or self.shapes[j][0] % 2:
                raise ValueError("a SwiGLU GEMV needs an even number of rows (gate and up halves)")
            if wtype == "bf16" or (wtype == "q4_0" and deq == 2):
                raise ValueError("the SwiGLU epilogue runs on Q8_0 chains and on q4_0 chains with int8 activations")
        for j in range(1, len(self.shapes)):
            if self.shapes[j][1] > self.out_len(j - 1):
                raise ValueError("a GEMV's k exceeds the previous GEMV's outputs")

        self.slots: List[GemvSlot] = []
        off = 0
        for layer in range(layers):
            for j, (n, k, _) in enumerate(self.shapes):
                wb = (wsg.q8_0_packed_bytes(n, k) if wtype == "q8_0" else
                      wsg.q4_0_packed_bytes(n, k) if wtype == "q4_0" else n * k * 2)
                self.slots.append(GemvSlot(layer, j, n, k, off, wb))
                off = _align(off + wb)
        self.weight_bytes_alloc = off
        self.weights = torch.empty(off, dtype=torch.uint8, device=device)
        k0 = self.shapes[0][1]
        self.inputs = torch.empty((layers, k0), dtype=torch.float32, device=device)
        for s in self.slots:
            s.y = torch.empty(self.out_len(s.index), dtype=torch.float32, device=device)
        # chain the inputs
        for i, s in enumerate(self.slots):
            if s.index == 0:
                s.x_ptr = self.inputs[s.layer].data_ptr()
            else:
                s.x_ptr = self.slots[i - 1].y.data_ptr()
        self.norm_before = tuple(sorted(set(int(j) for j in norm_before)))
        self.eps = float(eps)
        self.fused_norm = bool(fused_norm)
        if self.fused_norm and (wtype == "bf16" or (wtype == "q4_0" and deq == 2) or not self.norm_before):
            raise ValueError("fused_norm needs norm_before and a Q8_0 chain, or a q4_0 chain with int8 activations")
        self.norms: List[NormSlot] = []
        self.h0 = None
        self.gains = None
        if self.norm_before:
            self._lay_out_norms(device)
        self.xq = None
        if wtype == "q8_0" and requant == "separate":
            per = [_align(wsg.act_q8_0_bytes(k)) for _, k, _ in self.shapes]
            self.xq = torch.empty(layers * sum(per), dtype=torch.uint8, device=device)
            base = self.xq.data_ptr()
            for s in self.slots:
                s.xq_ptr = base
                base += per[s.index]
        self.plan = None

    def _lay_out_norms(self, device: str) -> None:
        hidden = self.shapes[self.norm_before[0]][1]
        nm = len(self.shapes)
        for j in self.norm_before:
            if not 0 <= j < nm or self.shapes[j][1] != hidden or self.shapes[j - 1][0] != hidden:
                raise ValueError("a normalized GEMV's k and the previous GEMV's rows must be the hidden size")
        self.hidden = hidden
        self.h0 = torch.zeros(hidden, dtype=torch.float32, device=device)
        count = self.layers * len(self.norm_before)
        self.gains = torch.ones((count, hidden), dtype=torch.float32, device=device)
        int8 = self.wtype in ("q8_0", "q4_0") and self.act_fmt() != wsg.ACT_F32
        h_in = self.h0.data_ptr()
        for i, s in enumerate(self.slots):
            if s.index not in self.norm_before:
                continue
            n = NormSlot(s.layer, s.index, h_in=h_in, g=self.gains[len(self.norms)].data_ptr())
            n.r = self.slots[i - 1].y.data_ptr() if i > 0 else 0
            n.h_out = torch.empty(hidden, dtype=torch.float32, device=device)
            n.y = torch.empty(hidden, dtype=torch.float32, device=device)
            if int8:
                n.yq = torch.empty(_align(wsg.act_q8_0_bytes(hidden)), dtype=torch.uint8, device=device)
            h_in = n.h_out.data_ptr()
            s.norm = n
            s.x_ptr = n.y.data_ptr()
            self.norms.append(n)

    def out_len(self, j: int) -> int:
        """Outputs of GEMV j of a layer: its rows, or half of them with SwiGLU."""
        n = self.shapes[j][0]
        return n // 2 if j in self.swiglu_at else n

    # ------------------------------------------------------------ sizes
    def algorithmic_weight_bytes(self) -> int:
        """Weight bytes per token at 34/32 (Q8_0), 18/32 (4-bit) or 2 (BF16) bytes per weight."""
        per = 0
        for n, k, _ in self.shapes:
            per += {"q8_0": n * (k // 32) * 34, "q4_0": n * (k // 32) * 18}.get(self.wtype, n * k * 2)
        return per * self.layers

    def act_fmt(self) -> int:
        if self.wtype == "bf16":
            return wsg.ACT_F32
        return wsg.act_fmt_for(self.deq, lm_head=False, fused_requant=(self.requant == "fused"))

    # ------------------------------------------------------------ filling
    def fill_weights(self, fill_rows: Callable[[int, int, int, int, torch.Tensor], None],
                     stream=None) -> None:
        """fill_rows(layer, matrix, part, rows, staging) writes rows x k f32
        values of one projection part into `staging` (a device tensor); they
        are then quantized (Q8_0) or rounded (BF16) into the part's row range."""
        kmax = max(k for _, k, _ in self.shapes)
        pmax = max(max(p) for _, _, p in self.shapes)
        staging = torch.empty(pmax * kmax, dtype=torch.float32, device=self.device)
        base = self.weights.data_ptr()
        for s in self.slots:
            _, k, parts = self.shapes[s.index]
            r0 = 0
            for pi, rows in enumerate(parts):
                buf = staging[: rows * k]
                fill_rows(s.layer, s.index, pi, rows, buf)
                if self.wtype == "q8_0":
                    dst = base + s.w_offset + r0 * wsg.q8_0_row_bytes(k)
                    wsg.quantize_q8_0_weights(buf, rows, k, dst, stream)
                elif self.wtype == "q4_0":
                    dst = base + s.w_offset + r0 * wsg.q4_0_row_bytes(k)
                    wsg.quantize_q4_0_weights(buf, rows, k, dst, stream)
                else:
                    dst = base + s.w_offset + r0 * k * 2
                    wsg.convert_bf16(buf, rows * k, dst, stream)
                r0 += rows
        torch.cuda.synchronize()
        del staging

    def set_inputs(self, x_rows: torch.Tensor) -> None:
        self.inputs.copy_(x_rows)

    def set_residual_input(self, h0: torch.Tensor, gains: torch.Tensor = None) -> None:
        """The residual stream entering layer 0 and (optionally) the gains of
        every norm call, in chain order ([layers * len(norm_before), hidden])."""
        self.h0.copy_(h0)
        if gains is not None:
            self.gains.copy_(gains)

    # ------------------------------------------------------------ calls
    def _slot_ops(self, s: GemvSlot) -> List[wsg.OpDesc]:
        w = self.weights.data_ptr() + s.w_offset
        if s.index in self.swiglu_at:
            nff = s.n // 2
            swiglu = wsg.op_gemv_q4_0_swiglu if self.wtype == "q4_0" else wsg.op_gemv_q8_0_swiglu
            if s.norm is not None:
                n = s.norm
                norm = wsg.op_residual_rmsnorm(n.h_in, n.r or None, n.g, self.hidden, self.eps, h_out=n.h_out,
                                               y=n.y, y_q8=n.yq)
                if n.yq is None:  # f32 activations (deq 2): the W8A16 SwiGLU GEMV reads y
                    return [norm, swiglu(w, nff, s.k, n.y, wsg.ACT_F32, s.y)]
                return [norm, swiglu(w, nff, s.k, n.yq, wsg.ACT_Q8_0, s.y)]
            if self.act_fmt() == wsg.ACT_Q8_0:
                return [wsg.op_quantize_act(s.x_ptr, s.k, s.xq_ptr),
                        swiglu(w, nff, s.k, s.xq_ptr, wsg.ACT_Q8_0, s.y)]
            return [swiglu(w, nff, s.k, s.x_ptr, self.act_fmt(), s.y)]
        pre = []
        if s.norm is not None and self.fused_norm:
            n = s.norm
            if self.wtype == "q4_0":
                return [wsg.op_gemv_q4_0_rmsnorm(w, s.n, s.k, n.h_in, n.r or None, n.g, self.eps, s.y,
                                                 h_out=n.h_out)]
            return [wsg.op_gemv_q8_0_rmsnorm(w, s.n, s.k, n.h_in, n.r or None, n.g, self.eps, s.y, h_out=n.h_out,
                                             act_fmt=wsg.ACT_F32 if self.act_fmt() == wsg.ACT_F32 else None)]
        if s.norm is not None:
            n = s.norm
            pre = [wsg.op_residual_rmsnorm(n.h_in, n.r or None, n.g, self.hidden, self.eps, h_out=n.h_out,
                                           y=n.y, y_q8=n.yq)]
            if n.yq is not None:
                gemv = wsg.op_gemv_q4_0 if self.wtype == "q4_0" else wsg.op_gemv_q8_0
                return pre + [gemv(w, s.n, s.k, n.yq, wsg.ACT_Q8_0, s.y)]
        if self.wtype == "bf16":
            return pre + [wsg.op_gemv_bf16(w, s.n, s.k, s.x_ptr, s.y)]
        if self.wtype == "q4_0":
            return [wsg.op_gemv_q4_0(w, s.n, s.k, s.x_ptr, wsg.ACT_F32 if self.deq == 2 else wsg.ACT_F32_REQUANT, s.y)]
        fmt = self.act_fmt()
        if pre:
            return pre + [wsg.op_gemv_q8_0(w, s.n, s.k, s.x_ptr, fmt, s.y)]
        if fmt == wsg.ACT_Q8_0:
            return [wsg.op_quantize_act(s.x_ptr, s.k, s.xq_ptr),
                    wsg.op_gemv_q8_0(w, s.n, s.k, s.xq_ptr, wsg.ACT_Q8_0, s.y)]
        return [wsg.op_gemv_q8_0(w, s.n, s.k, s.x_ptr, fmt, s.y)]

    def ops(self) -> List[wsg.OpDesc]:
        """The token's calls in order.  A layer's first call is marked as
        depending on everything before it: in a model its input comes from
        the previous layer's output (through operators outside this stream),
        so no plan may start it early."""
        out = []
        per_layer = len(self.slots) // self.layers
        for i, s in enumerate(self.slots):
            ops = self._slot_ops(s)
            if i > 0 and i % per_layer == 0:
                ops[0].flags |= wsg.OP_AFTER_ALL
            out.extend(ops)
        return out

    def run_slot(self, i: int, stream=None) -> None:
        """One GEMV of the chain, eagerly: the same calls the plan captured."""
        for op in self._slot_ops(self.slots[i]):
            if op.op == wsg.OP_GEMV_BF16:
                wsg.gemv_bf16(op.w, op.n, op.k, op.x, op.y, stream=stream)
            elif op.op == wsg.OP_QUANTIZE_ACT:
                wsg.quantize_act_q8_0(op.x, op.k, op.y, stream=stream)
            elif op.op == wsg.OP_RESIDUAL_RMSNORM:
                wsg.residual_rmsnorm_q8_0(op.x, op.r, op.w, op.k, op.eps, h_out=op.h_out, y=op.y, y_q8=op.y_q8,
                                          stream=stream)
            elif op.op == wsg.OP_GEMV_Q4_0:
                wsg.gemv_q4_0(op.w, op.n, op.k, op.x, op.act_fmt, op.y, stream=stream)
            elif op.op == wsg.OP_GEMV_Q8_0_SWIGLU:
                wsg.gemv_q8_0_swiglu(op.w, op.n, op.k, op.x, op.act_fmt, op.y, stream=stream)
            elif op.op == wsg.OP_GEMV_Q4_0_SWIGLU:
                wsg.gemv_q4_0_swiglu(op.w, op.n, op.k, op.x, op.act_fmt, op.y, stream=stream)
            elif op.op in (wsg.OP_GEMV_Q8_0_RMSNORM, wsg.OP_GEMV_Q4_0_RMSNORM):
                f = (wsg.gemv_q4_0_rmsnorm if op.op == wsg.OP_GEMV_Q4_0_RMSNORM else
                     wsg.gemv_q8_0_rmsnorm_f32 if op.act_fmt == wsg.ACT_F32 else wsg.gemv_q8_0_rmsnorm)
                f(op.w, op.n, op.k, op.x, op.r, op.g, op.eps, op.y, h_out=op.h_out, stream=stream)
            else:
                wsg.gemv_q8_0(op.w, op.n, op.k, op.x, op.act_fmt, op.y, stream=stream)

    def run_eager(self, stream=None) -> None:
        for i in range(len(self.slots)):
            self.run_slot(i, stream)

    def capture(self, stream=None, persistent: bool = False) -> wsg.Plan:
        """One hipGraph per token: a node per call, or (persistent=True, Q8_0
        chains with fused requantization or f32 activations) one resident
        kernel for the whole token."""
        if self.plan is not None:
            self.plan.destroy()
        self.plan = wsg.Plan(self.ops(), stream=stream, persistent=persistent)
        return self.plan

    def launch(self, stream=None) -> None:
        if self.plan is None:
            self.capture(stream)
        self.plan.launch(stream)

    def outputs(self):
        return [s.y for s in self.slots]

    def weight_ptr(self, i: int) -> int:
        return self.weights.data_ptr() + self.slots[i].w_offset

    def close(self) -> None:
        if self.plan is not None:
            self.plan.destroy()
            self.plan = None


class DecodeStep:
    """One whole batch-1 decode step on the device, captured as one graph
    (GPU Kernel Lab, "Decode integration": fixed token/position buffers,
    ..., the LM-head GEMV + argmax + token/position update, fixed-address
    graph replay; emit_qwen38_generate, "Where the speed comes from",
    item 2: the sampled token and the position advance on the device, so no
    replay needs a host round trip):

      embed_gather(token) -> residual stream h0
      -> the layer chain (residual add + RMSNorm before the attention and
         MLP inputs, fused into the attention-input GEMV; SwiGLU on gate+up)
      -> residual add + final RMSNorm -> LM-head GEMV + argmax -> token
      -> token_advance(token, history, pos)

    Each replay decodes one token; history holds the tokens decoded so far.
    Attention and the other non-GEMV operators are not part of this path:
    the layer chain is the GEMV stream (q/k/v -> o_proj reads the first
    rows of the qkv output).  wtype is the layers' weight format ("q8_0" or
    "q4_0"); the embedding table and the LM head stay Q8_0.

    deq (emit_qwen38_generate, "Where the speed comes from", the deq
    paragraph) picks where activations are quantized: 0 = every GEMV takes
    int8 activations; 1 = the layers do, the LM head takes the f32 final
    normalized vector; 2 = every Q8_0 GEMV takes f32 activations (the fused
    norm GEMVs' f32 form, the W8A16 SwiGLU GEMV, the dequantizing down
    projection and LM head), so no activation is quantized anywhere.  q4_0
    layers run deq 0 or 1."""

    def __init__(self, shapes, layers: int, vocab: int, capacity: int = 1024, device: str = "cuda",
                 eps: float = 1e-6, wtype: str = "q8_0", deq: int = 0):
        if wtype not in ("q8_0", "q4_0"):
            raise ValueError("the decode step's layers are Q8_0 or q4_0")
        if deq not in (0, 1, 2) or (wtype == "q4_0" and deq == 2):
            raise ValueError("deq is 0, 1 or 2 (q4_0 layers: 0 or 1)")
        self.deq = deq
        self.head_act = wsg.ACT_Q8_0 if deq == 0 else wsg.ACT_F32
        self.chain = TokenStream(shapes, layers, wtype, deq=2 if deq == 2 else 0, device=device,
                                 norm_before=(0, 2), eps=eps, fused_norm=True, swiglu_at=(2,))
        self.hidden = self.chain.hidden
        self.vocab = int(vocab)
        self.capacity = int(capacity)
        self.eps = float(eps)
        rb = wsg.q8_0_packed_bytes(self.vocab, self.hidden)
        self.embedding = torch.empty(rb, dtype=torch.uint8, device=device)
        self.lm_head = torch.empty(rb, dtype=torch.uint8, device=device)
        self.final_gain = torch.ones(self.hidden, dtype=torch.float32, device=device)
        self.final_h = torch.empty(self.hidden, dtype=torch.float32, device=device)
        self.final_y = torch.empty(self.hidden, dtype=torch.float32, device=device)
        self.final_q8 = torch.empty(_align(wsg.act_q8_0_bytes(self.hidden)), dtype=torch.uint8, device=device)
        self.logits = torch.empty(self.vocab, dtype=torch.float32, device=device)
        self.ws = torch.empty(wsg.argmax_ws_bytes(), dtype=torch.uint8, device=device)
        self.token = torch.zeros(1, dtype=torch.int32, device=device)
        self.pos = torch.zeros(1, dtype=torch.int32, device=device)
        self.history = torch.full((max(self.capacity, 1),), -1, dtype=torch.int32, device=device)
        self.plan = None

    def fill_table(self, table: torch.Tensor, fill_rows: Callable[[int, torch.Tensor], None],
                   rows_per_call: int = 8192) -> None:
        """Quantize a vocab x hidden table into `table` (embedding or LM
        head): fill_rows(first_row, staging f32 [rows, hidden])."""
        staging = torch.empty((rows_per_call, self.hidden), dtype=torch.float32, device=table.device)
        row_bytes = wsg.q8_0_row_bytes(self.hidden)
        for r0 in range(0, self.vocab, rows_per_call):
            rows = min(rows_per_call, self.vocab - r0)
            fill_rows(r0, staging[:rows])
            wsg.quantize_q8_0_weights(staging[:rows], rows, self.hidden, table[r0 * row_bytes:])
        torch.cuda.synchronize()

    def final_q8_or_none(self):
        """The final norm's Q8_0 output, written only when the LM head reads it."""
        return self.final_q8 if self.head_act == wsg.ACT_Q8_0 else None

    def head_input(self) -> torch.Tensor:
        """The LM head's activation: the final norm's Q8_0 codes (deq 0) or
        its f32 output (deq 1 and 2)."""
        return self.final_q8 if self.head_act == wsg.ACT_Q8_0 else self.final_y

    def reset(self, first_token: int) -> None:
        """Start a sequence: the current token, an empty history, position 0."""
        self.token.fill_(int(first_token))
        self.pos.zero_()
        self.history.fill_(-1)

    def ops(self) -> List[wsg.OpDesc]:
        chain = self.chain
        last = chain.slots[-1]
        h_last = chain.norms[-1].h_out
        return ([wsg.op_embed_gather(self.embedding, wsg.W_Q8_0, self.vocab, self.hidden, self.token, chain.h0)]
                + chain.ops()
                + [wsg.op_residual_rmsnorm(h_last, last.y, self.final_gain, self.hidden, self.eps,
                                           h_out=self.final_h, y=self.final_y, y_q8=self.final_q8_or_none()),
                   wsg.op_lm_head_argmax(self.lm_head, wsg.W_Q8_0, self.vocab, self.hidden, self.head_input(),
                                         self.head_act, self.ws, self.ws.numel(), self.token,
                                         debug_logits=self.logits),
                   wsg.op_token_advance(self.token, self.history, self.capacity, self.pos)])

    def run_eager(self, stream=None) -> None:
        """One step through the same calls, one at a time."""
        wsg.embed_gather(self.embedding, wsg.W_Q8_0, self.vocab, self.hidden, self.token, self.chain.h0,
                         stream=stream)
        self.chain.run_eager(stream)
        last = self.chain.slots[-1]
        wsg.residual_rmsnorm_q8_0(self.chain.norms[-1].h_out, last.y, self.final_gain, self.hidden, self.eps,
                                  h_out=self.final_h, y=self.final_y, y_q8=self.final_q8_or_none(), stream=stream)
        wsg.lm_head_argmax(self.lm_head, wsg.W_Q8_0, self.vocab, self.hidden, self.head_input(), self.head_act,
                           self.ws, self.ws.numel(), self.token, self.logits, stream=stream)
        wsg.token_advance(self.token, self.history, self.capacity, self.pos, stream=stream)

    def capture(self, stream=None) -> wsg.Plan:
        if self.plan is not None:
            self.plan.destroy()
        self.plan = wsg.Plan(self.ops(), stream=stream)
        return self.plan

    def launch(self, stream=None) -> None:
        if self.plan is None:
            self.capture(stream)
        self.plan.launch(stream)

    def close(self) -> None:
        if self.plan is not None:
            self.plan.destroy()
            self.plan = None
        self.chain.close()
