"""The five synthetic workloads: shapes, value distributions and seeds.

Shapes are rows x K (N x K); W is row-major and y = W.x is f32[N].
Concatenated projections are listed with their parts (rows of each part, in
stacking order).  Only shapes, ids and seeds live here: no arithmetic.

Sources for the shapes (all batch-1 decode):
  * single Q8_0 GEMV 1024x1024 with outlier activations;
  * Qwen3-0.6B-shaped BF16 decode layer (GPU Kernel Lab, "Decode
    integration");
  * Qwen3-8B-shaped Q8_0 decode (qwen3-8b-rtx4080-cutedsl, "GQA + QK-Norm":
    32 query heads, 8 KV heads);
  * lm_head 151936x4096 with planted ties;
  * dense 27B-scale Q8_0 stream, 64 layers; the qkvz (16384 rows) and gate+up
    (34816 rows) widths are those of emit_qwen38_generate, "Where the speed
    comes from", item 1.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

SEED_BASE = 0x5EED0000
WEIGHT_SIGMA = 0.02

Q8_BYTES_PER_WEIGHT = 34.0 / 32.0
BF16_BYTES_PER_WEIGHT = 2.0


@dataclass(frozen=True)
class Matrix:
    name: str
    n: int
    k: int
    parts: Tuple[int, ...]  # row counts of the stacked projections

    def __post_init__(self):
        assert sum(self.parts) == self.n, (self.name, self.parts, self.n)


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    wtype: str  # "q8_0" or "bf16"
    layers: int
    matrices: Tuple[Matrix, ...]
    description: str
    deq_modes: Tuple[int, ...] = ()

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    def bytes_per_weight(self) -> float:
        return Q8_BYTES_PER_WEIGHT if self.wtype == "q8_0" else BF16_BYTES_PER_WEIGHT

    def weight_bytes_per_layer(self) -> int:
        per = 0
        for m in self.matrices:
            if self.wtype == "q8_0":
                per += m.n * (m.k // 32) * 34
            else:
                per += m.n * m.k * 2
        return per

    def weight_bytes(self) -> int:
        return self.layers * self.weight_bytes_per_layer()

    def gemvs_per_token(self) -> int:
        return self.layers * len(self.matrices)


def weight_tensor_id(layer: int, matrix: int, part: int) -> int:
    """Tensor id of one projection part; its element (r, c) is draw r*K + c."""
    return ((layer * 16 + matrix) * 8 + part) * 2


def activation_tensor_id(layer: int) -> int:
    """Tensor id of layer `layer`'s input activation (the next id, +1, picks
    its outlier positions)."""
    return 1_000_000 + 4 * layer


# Inputs of the chained token (residual stream + RMSNorm between GEMVs): the
# residual stream entering layer 0 ~N(0,1) (an embedding row) and the gain
# of every norm call, 1 + N(0, GAIN_SIGMA), in chain order.
GAIN_SIGMA = 0.1
RMSNORM_EPS = 1e-6
RESIDUAL_TENSOR_ID = 2_000_000
# embedding table and LM head of a whole decode step
EMBEDDING_TENSOR_ID = 3_000_000
LM_HEAD_TENSOR_ID = 3_000_001


def gain_tensor_id(i: int) -> int:
    return 2_000_002 + 2 * i


Q8_SINGLE = Workload(
    0, "q8_single_1024x1024", "q8_0", 1,
    (Matrix("w", 1024, 1024, (1024,)),),
    "Single Q8_0 GEMV 1024x1024; weights ~N(0,0.02); x ~N(0,1) with 1% of entries x20",
    deq_modes=(0, 2),
)

QWEN3_0P6B_BF16 = Workload(
    1, "qwen3_0.6b_bf16_28L", "bf16", 28,
    (
        Matrix("qkv", 4096, 1024, (2048, 1024, 1024)),
        Matrix("o_proj", 1024, 2048, (1024,)),
        Matrix("gate_up", 6144, 1024, (3072, 3072)),
        Matrix("down", 1024, 3072, (1024,)),
    ),
    "Qwen3-0.6B-shaped BF16 decode, 28 layers, RMS-scaled activations",
)

QWEN3_8B_Q8 = Workload(
    2, "qwen3_8b_q8_0_36L", "q8_0", 36,
    (
        Matrix("qkv", 6144, 4096, (4096, 1024, 1024)),
        Matrix("o_proj", 4096, 4096, (4096,)),
        Matrix("gate_up", 24576, 4096, (12288, 12288)),
        Matrix("down", 4096, 12288, (4096,)),
    ),
    "Qwen3-8B-shaped Q8_0 decode, 36 layers, int8 per-block activations",
    deq_modes=(0,),
)

LM_HEAD = Workload(
    3, "lm_head_151936x4096", "both", 1,
    (Matrix("lm_head", 151936, 4096, (151936,)),),
    "lm_head 151936x4096 in BF16 and Q8_0 with fused on-device argmax and planted ties",
    deq_modes=(0, 1, 2),
)

DENSE27B_Q8 = Workload(
    4, "dense27b_q8_0_64L", "q8_0", 64,
    (
        Matrix("qkvz", 16384, 5120, (16384,)),
        Matrix("out", 5120, 8192, (5120,)),
        Matrix("gate_up", 34816, 5120, (17408, 17408)),
        Matrix("down", 5120, 17408, (5120,)),
    ),
    "27B-scale synthetic Q8_0 token stream, 64 layers, one hipGraph replay",
    deq_modes=(0, 2),
)

ALL: List[Workload] = [Q8_SINGLE, QWEN3_0P6B_BF16, QWEN3_8B_Q8, LM_HEAD, DENSE27B_Q8]


def chain_input_len(w: Workload, m_index: int) -> int:
    """K of matrix m_index; its input is the previous GEMV's output
    truncated to K (the first GEMV of a layer reads the layer input)."""
    return w.matrices[m_index].k
