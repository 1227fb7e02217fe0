"""Seeded synthetic inputs for the TP-MLP workloads.

This module holds the workload table and the seeded input generators that
both the HIP path (through the tests and the benchmark) and the fp64 oracle
receive.  It holds none of the method's arithmetic: it draws Gaussian
numbers, rounds them to the storage type, and returns them.

Recipe (identical for every workload):
  * generator  numpy.random.default_rng(seed) (PCG64);
  * draw order X (or x), then A, then B, each as standard_normal(shape,
    float32), then multiplied by its standard deviation in float32;
  * bf16 workloads round each float32 value to the nearest bfloat16 (ties to
    even) here, so the float32 arrays returned hold exactly the values the GPU
    receives, and the oracle upcasts them to float64 exactly;
  * dense i.i.d. values, no sparsity or structure.

The shapes follow the workloads of the pages (tokens M = b*s rows of width D,
A of shape (D, F), B of shape (F, D), N shards): the worked example of
"Tensor-Parallel MLP (Megatron)" (section "The split", "Example"), a small
fp32 case, three bf16 sizes, and the FFN half of the Post-LN block of
"LLM Lab Notes 06" at s in {128, 256, 512}, with the LayerNorm before the
MLP as that page's code places it and after the residual as its prose does
(the same inputs for both).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# The worked example printed by "Tensor-Parallel MLP (Megatron)", section
# "The split", paragraph "Example": one token, D = 2, F = 4, N = 2.
WORKED_X = [[1.0, 2.0]]
WORKED_A = [[1.0, 0.0, -1.0, 2.0], [0.0, 1.0, 1.0, -1.0]]
WORKED_B = [[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [2.0, 0.0]]


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    D: int
    F: int
    n: int
    dtype: str              # "f32" or "bf16": storage of X, A, B, H and Y
    sx: float
    sa: float
    sb: float
    seed: int
    layernorm: bool = False
    residual: bool = False
    note: str = ""
    layernorm_after: bool = False

    @property
    def flops(self) -> int:
        """4*M*D*F: two GEMMs of 2*M*D*F each."""
        return 4 * self.M * self.D * self.F


WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 16, 64, 256, 2, "f32", 1.0, 1.0 / 8, 1.0 / 16, 1001,
                         note="X[16,64]~N(0,1), A~N(0,1/64), B~N(0,1/256), N=2"),
    "mlp_h1024_bf16": Workload("mlp_h1024_bf16", 4 * 512, 1024, 4096, 4, "bf16", 1.0, 0.02, 0.02, 1002,
                               note="M=b*s=4*512, D=1024, F=4096, N=4"),
    "mlp_h4096_bf16": Workload("mlp_h4096_bf16", 8 * 2048, 4096, 16384, 8, "bf16", 1.0, 0.02, 0.02, 1003,
                               note="M=8*2048, D=4096, F=16384, N=8 (headline MFMA-roofline size)"),
    "rank_h8192_bf16": Workload("rank_h8192_bf16", 4 * 2048, 8192, 32768 // 8, 1, "bf16", 1.0, 0.02, 0.02, 1004,
                                note="one TP rank of a wide MLP: F_local=32768/8=4096, single shard"),
}
for _s in (128, 256, 512):
    WORKLOADS[f"postln_s{_s}_bf16"] = Workload(
        f"postln_s{_s}_bf16", 8 * _s, 1024, 4096, 4, "bf16", 1.0, 0.02, 0.02, 1005 + _s,
        layernorm=True, residual=True,
        note=f"Post-LN FFN half: LayerNorm -> TP-MLP -> x + Y, b=8, s={_s}, h=1024")
    # the same inputs with the Norm moved after the residual (the order the
    # prose of that page describes): LayerNorm(x + TP-MLP(x))
    WORKLOADS[f"lnafter_s{_s}_bf16"] = Workload(
        f"lnafter_s{_s}_bf16", 8 * _s, 1024, 4096, 4, "bf16", 1.0, 0.02, 0.02, 1005 + _s,
        residual=True, layernorm_after=True,
        note=f"FFN half, Norm after the residual: LayerNorm(x + TP-MLP(x)), b=8, s={_s}, h=1024")

HEADLINE = "mlp_h4096_bf16"


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Inputs here are finite Gaussian draws, so NaN handling is not needed.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    hi = ((bits + bias) >> 16).astype(np.uint32)
    return (hi << 16).view(np.float32)


def _draw(rng: np.random.Generator, shape, sigma: float, dtype: str) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(sigma)
    if dtype == "bf16":
        a = round_to_bf16(a)
    return a


@dataclass
class Inputs:
    X: np.ndarray
    A: np.ndarray
    B: np.ndarray
    workload: Optional[Workload] = None
    extra: dict = field(default_factory=dict)


def make_inputs(w: Workload, M: Optional[int] = None) -> Inputs:
    """Seeded X[M,D], A[D,F], B[F,D] (float32 arrays holding storage-type values)."""
    rng = np.random.default_rng(w.seed)
    M = w.M if M is None else M
    X = _draw(rng, (M, w.D), w.sx, w.dtype)
    A = _draw(rng, (w.D, w.F), w.sa, w.dtype)
    B = _draw(rng, (w.F, w.D), w.sb, w.dtype)
    return Inputs(X, A, B, w)


def worked_example() -> Inputs:
    return Inputs(np.array(WORKED_X, np.float32), np.array(WORKED_A, np.float32),
                  np.array(WORKED_B, np.float32))


def random_case(M: int, D: int, F: int, seed: int, dtype: str = "f32",
                sx: float = 1.0, sa: Optional[float] = None, sb: Optional[float] = None) -> Inputs:
    """Seeded case of arbitrary shape, scaled like the tiny workload (sigma 1/sqrt(fan-in))."""
    rng = np.random.default_rng(seed)
    sa = (1.0 / np.sqrt(D)) if sa is None else sa
    sb = (1.0 / np.sqrt(F)) if sb is None else sb
    return Inputs(_draw(rng, (M, D), sx, dtype), _draw(rng, (D, F), sa, dtype),
                  _draw(rng, (F, D), sb, dtype))


# ---------------------------------------------------------------------------
# the attention half of the block
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class AttnWorkload:
    name: str
    batch: int
    seq: int
    hidden: int
    heads: int
    p: int
    sx: float
    sw: float
    seed: int
    note: str = ""

    @property
    def M(self) -> int:
        return self.batch * self.seq

    @property
    def flops(self) -> int:
        """Projections 2*M*h*3h, scores and P V 2 * 2*b*s*s*h (every head), without W^O."""
        return 2 * self.M * self.hidden * 3 * self.hidden + 4 * self.batch * self.seq * self.seq * self.hidden


# The block of "LLM Lab Notes 06" (b = 8 as for its FFN, s in {128, 256, 512},
# 4 ranks); the pages give no head count, so h = 1024 as 16 heads of 64.
ATTN_WORKLOADS: Dict[str, AttnWorkload] = {}
for _s in (128, 256, 512):
    ATTN_WORKLOADS[f"attn_s{_s}_bf16"] = AttnWorkload(
        f"attn_s{_s}_bf16", 8, _s, 1024, 16, 4, 1.0, 0.02, 2005 + _s,
        note=f"attention half: LayerNorm -> QKV -> softmax(QK^T/8)V per head -> cat -> x + attn, b=8, s={_s}")


@dataclass
class AttnInputs:
    x: np.ndarray
    Wq: np.ndarray
    Wk: np.ndarray
    Wv: np.ndarray
    Wo: np.ndarray


def make_attn_inputs(w: AttnWorkload) -> AttnInputs:
    """Seeded x[M,h], then W^Q, W^K, W^V, W^O [h,h] (bf16 values in float32 arrays)."""
    return attn_case(w.batch, w.seq, w.hidden, w.seed, w.sx, w.sw)


def attn_case(batch: int, seq: int, hidden: int, seed: int, sx: float = 1.0,
              sw: Optional[float] = None) -> AttnInputs:
    """Seeded attention inputs of any shape; sw defaults to 1/sqrt(h)."""
    rng = np.random.default_rng(seed)
    sw = (1.0 / np.sqrt(hidden)) if sw is None else sw
    x = _draw(rng, (batch * seq, hidden), sx, "bf16")
    W = [_draw(rng, (hidden, hidden), sw, "bf16") for _ in range(4)]
    return AttnInputs(x, *W)
