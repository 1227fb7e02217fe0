"""fp64 CPU oracle for the Megatron tensor-parallel MLP forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library and imports
nothing from it.

What it computes (sources are the four web pages on Megatron tensor
parallelism; each function names the passage it follows):

    Y = sum_i GeLU_tanh(X A_i) B_i

with A split by columns into n contiguous blocks A_i and B split by the
matching rows into B_i ("Tensor-Parallel MLP (Megatron)", scratchllm,
sections "The problem", "The split", "Requirements").  The optional Post-LN
FFN half of a block, out = x + TP-MLP(LayerNorm(x)), follows the code
walkthrough of "LLM Lab Notes 06: Building a Megatron-Style Transformer
Block from Scratch", section 2, markers 5 to 7.

Everything is evaluated in float64 with plain numpy matmuls, in the order the
pages state the steps; there is no blocking, fusion or reordering.  A second,
pure-Python implementation (``*_loops``) exists for tiny inputs so that the
numpy version can be checked against code that uses no numpy at all.

Every function here is pinned by tests in ``tests/test_oracle.py`` against
the values the pages print for their worked example, closed forms,
invariants and library special cases.  The readings taken where the pages
are silent (LayerNorm epsilon, residual added once after the shard sum)
are stated at the function that takes them.
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

# Constants of the GPT-2 tanh approximation ("Tensor-Parallel MLP
# (Megatron)", section "GeLU", the displayed equation).
SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_CUBIC = 0.044715

# LayerNorm epsilon.  The block code calls F.layer_norm(x, (hidden,)) with no
# further arguments ("LLM Lab Notes 06", section 2, markers 2 and 5); the plain
# reading of that call is PyTorch's default eps = 1e-5, biased variance and
# no affine weight or bias.  The pages themselves do not print a value.
LN_EPS = 1e-5


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# numpy fp64 oracle
# --------------------------------------------------------------------------

def gelu(x) -> np.ndarray:
    """tanh-GeLU, elementwise, in float64.

    "Tensor-Parallel MLP (Megatron)", section "GeLU": GeLU(x) is approximated
    by one half of x times (1 + tanh u), where the helper value u is
    sqrt(2/pi) times (x + 0.044715 x^3).  Evaluated exactly in that form.
    """
    x = _f64(x)
    with np.errstate(over="ignore", invalid="ignore"):
        u = SQRT_2_OVER_PI * (x + GELU_CUBIC * (x * x * x))
        return 0.5 * x * (1.0 + np.tanh(u))


def shard_mlp(A, B, n: int) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Return the n pairs (A_i, B_i).

    "Tensor-Parallel MLP (Megatron)", sections "The split" and
    "Requirements": GPU i receives columns iF/n .. (i+1)F/n - 1 of A and the
    same range of rows of B; F must be divisible by n ("What to implement").
    """
    A = _f64(A)
    B = _f64(B)
    if A.ndim != 2 or B.ndim != 2:
        raise ValueError("A and B must be matrices")
    D, F = A.shape
    if B.shape != (F, D):
        raise ValueError(f"B must have shape (F, D) = ({F}, {D}), got {B.shape}")
    if n <= 0 or n > F or F % n != 0:
        raise ValueError(f"F={F} must be divisible by n={n} with 0 < n <= F")
    w = F // n
    return [(A[:, i * w:(i + 1) * w], B[i * w:(i + 1) * w, :]) for i in range(n)]


def shard_outputs(X, shards: Sequence[Tuple[np.ndarray, np.ndarray]]):
    """Per-GPU intermediates and partial outputs, in shard order.

    "Tensor-Parallel MLP (Megatron)", section "The split": H_i = GeLU(X A_i)
    (bullet 1) and Y_i = H_i B_i, already of the full output shape (bullet 2).
    Returns (H_list, Y_list).
    """
    X = _f64(X)
    H_list, Y_list = [], []
    for A_i, B_i in shards:
        H_i = gelu(X @ _f64(A_i))
        Y_list.append(H_i @ _f64(B_i))
        H_list.append(H_i)
    return H_list, Y_list


def tp_mlp(X, shards: Sequence[Tuple[np.ndarray, np.ndarray]]) -> np.ndarray:
    """Sum of the partial outputs (the simulated all-reduce).

    "Tensor-Parallel MLP (Megatron)", section "The split", bullet 3, and
    "What to implement": Y = sum_i Y_i, each Y_i computed from its own
    (A_i, B_i) only.  The sum runs in ascending i; the pages fix no order.
    """
    _, Y_list = shard_outputs(X, shards)
    Y = np.zeros_like(Y_list[0])
    for Y_i in Y_list:
        Y = Y + Y_i
    return Y


def layer_norm(x, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last (hidden) axis with no affine parameters.

    "LLM Lab Notes 06", section 2, markers 2 and 5: F.layer_norm(x, (hidden,)).
    mean and biased variance over the hidden axis; (x - mean) / sqrt(var + eps).
    """
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def post_ln_ffn(x, shards, eps: float = LN_EPS) -> np.ndarray:
    """FFN half of the Post-LN block: out = x + TP-MLP(LayerNorm(x)).

    "LLM Lab Notes 06", section 2: marker 5 normalises x, marker 6 runs the
    column- then row-parallel FFN and all-reduces its output, marker 7 adds
    the residual.  The residual is the un-normalised x and is added once,
    after the sum over shards (the all-reduce comes before the residual in
    that code).
    """
    x = _f64(x)
    return x + tp_mlp(layer_norm(x, eps), shards)


# --------------------------------------------------------------------------
# pure-Python oracle (no numpy arithmetic), for tiny inputs only
# --------------------------------------------------------------------------

def gelu_scalar(x: float) -> float:
    """Scalar tanh-GeLU with math.tanh ("Tensor-Parallel MLP (Megatron)", "GeLU")."""
    x = float(x)
    u = SQRT_2_OVER_PI * (x + GELU_CUBIC * x * x * x)
    return 0.5 * x * (1.0 + math.tanh(u))


def _matmul_loops(P: List[List[float]], Q: List[List[float]]) -> List[List[float]]:
    rows, inner, cols = len(P), len(Q), len(Q[0])
    out = [[0.0] * cols for _ in range(rows)]
    for r in range(rows):
        Pr = P[r]
        orow = out[r]
        for k in range(inner):
            p = Pr[k]
            Qk = Q[k]
            for c in range(cols):
                orow[c] += p * Qk[c]
    return out


def tp_mlp_loops(X, A, B, n: int):
    """Pure-Python version of the whole method on lists of floats.

    Same steps as the numpy oracle ("The split" bullets 1 to 3): slice the
    column block of A and the row block of B for each i, form GeLU(X A_i)
    entry by entry, multiply by B_i and accumulate the partials in order.
    Returns (Y, partials), both as nested lists.
    """
    X = [[float(v) for v in row] for row in X]
    A = [[float(v) for v in row] for row in A]
    B = [[float(v) for v in row] for row in B]
    D, F = len(A), len(A[0])
    if len(B) != F or any(len(r) != D for r in B):
        raise ValueError("B must be F x D")
    if n <= 0 or n > F or F % n:
        raise ValueError("F must be divisible by n")
    w = F // n
    M = len(X)
    Y = [[0.0] * D for _ in range(M)]
    partials = []
    for i in range(n):
        A_i = [row[i * w:(i + 1) * w] for row in A]
        B_i = B[i * w:(i + 1) * w]
        S_i = _matmul_loops(X, A_i)
        H_i = [[gelu_scalar(v) for v in row] for row in S_i]
        Y_i = _matmul_loops(H_i, B_i)
        partials.append(Y_i)
        for r in range(M):
            for c in range(D):
                Y[r][c] += Y_i[r][c]
    return Y, partials


def layer_norm_loops(x, eps: float = LN_EPS):
    """Pure-Python LayerNorm over each row (no affine), for tiny inputs."""
    out = []
    for row in x:
        row = [float(v) for v in row]
        h = len(row)
        mu = sum(row) / h
        var = sum((v - mu) ** 2 for v in row) / h
        inv = 1.0 / math.sqrt(var + eps)
        out.append([(v - mu) * inv for v in row])
    return out
