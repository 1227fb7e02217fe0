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
Block from Scratch", section 2, markers 5 to 7; the other placement that
page describes, out = LayerNorm(x + TP-MLP(x)) (residual first, then the
Norm), is ``norm_after_ffn``.

The backward pass of the same MLP (the gradients of a loss L given
dY = dL/dY) follows from the chain rule applied to the forward as defined
above; the pages print no backward formulas, but "LLM Lab Notes 06"
(section 2, marker 1, and the ledger of section 3) state that backward
all-reduces the gradient at the same point the forward all-reduced, which
here is the sum over shards of the input gradient.

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


def norm_after_ffn(x, shards, eps: float = LN_EPS) -> np.ndarray:
    """FFN half with the LayerNorm after the residual: out = LayerNorm(x + TP-MLP(x)).

    "LLM Lab Notes 06", section 2, the note on markers 2 and 5: the prose
    describes the Post-LN order of the original Transformer, the residual
    added first and the LayerNorm applied to the sum, and says the Pre-LN
    order (normalise first, the code as printed and ``post_ln_ffn`` above)
    differs only in where the Norm and the residual sit; section 5,
    takeaway 2, contrasts the two.  Reading: the TP-MLP sees the raw x, the
    shard sum (the all-reduce) comes before the residual as in the code,
    and the LayerNorm is the same no-affine one over the hidden axis.
    """
    x = _f64(x)
    return layer_norm(x + tp_mlp(x, shards), eps)


def gelu_grad(x) -> np.ndarray:
    """Derivative of the tanh-GeLU of "Tensor-Parallel MLP (Megatron)",
    section "GeLU", in float64.

    With u = sqrt(2/pi) (x + 0.044715 x^3) and g(x) = x (1 + tanh u) / 2,
    the product and chain rules give
    g'(x) = (1 + tanh u) / 2 + x (1 - tanh^2 u) sqrt(2/pi) (1 + 3 * 0.044715 x^2) / 2.
    """
    x = _f64(x)
    with np.errstate(over="ignore", invalid="ignore"):
        u = SQRT_2_OVER_PI * (x + GELU_CUBIC * (x * x * x))
        t = np.tanh(u)
        du = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_CUBIC * (x * x))
        return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du


def tp_mlp_backward(X, shards: Sequence[Tuple[np.ndarray, np.ndarray]], dY):
    """Gradients of the TP-MLP given dY = dL/dY, shard by shard.

    Forward ("Tensor-Parallel MLP (Megatron)", "The split"): S_i = X A_i,
    H_i = GeLU(S_i), Y = sum_i H_i B_i.  The chain rule gives, for each i,
        dB_i = H_i^T dY,   dS_i = (dY B_i^T) * GeLU'(S_i),   dA_i = X^T dS_i,
    and the input gradient dX = sum_i dS_i A_i^T, summed over shards in
    ascending i: the backward all-reduce of "LLM Lab Notes 06", section 2,
    marker 1 (its autograd function all-reduces the incoming gradient) and
    the backward row of the ledger in section 3.
    Returns (dX, [dA_i], [dB_i]).
    """
    X = _f64(X)
    dY = _f64(dY)
    dX = np.zeros_like(X)
    dA_list, dB_list = [], []
    for A_i, B_i in shards:
        A_i = _f64(A_i)
        B_i = _f64(B_i)
        S_i = X @ A_i
        H_i = gelu(S_i)
        dB_list.append(H_i.T @ dY)
        dS_i = (dY @ B_i.T) * gelu_grad(S_i)
        dA_list.append(X.T @ dS_i)
        dX = dX + dS_i @ A_i.T
    return dX, dA_list, dB_list


def tp_mlp_backward_full(X, A, B, n: int, dY):
    """tp_mlp_backward over shard_mlp(A, B, n), with the per-shard weight
    gradients placed back where their shards came from: dA (D x F) has dA_i
    in columns iF/n .. (i+1)F/n - 1, dB (F x D) has dB_i in those rows."""
    dX, dA_list, dB_list = tp_mlp_backward(X, shard_mlp(A, B, n), dY)
    return dX, np.concatenate(dA_list, axis=1), np.concatenate(dB_list, axis=0)


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


def norm_after_ffn_loops(x, A, B, n: int, eps: float = LN_EPS):
    """Pure-Python version of norm_after_ffn on nested lists (tiny inputs)."""
    Y, _ = tp_mlp_loops(x, A, B, n)
    z = [[float(a) + float(b) for a, b in zip(xr, yr)] for xr, yr in zip(x, Y)]
    return layer_norm_loops(z, eps)


def gelu_grad_scalar(x: float) -> float:
    """Scalar derivative of the tanh-GeLU (same formula as gelu_grad)."""
    x = float(x)
    u = SQRT_2_OVER_PI * (x + GELU_CUBIC * x * x * x)
    t = math.tanh(u)
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_CUBIC * x * x)


def tp_mlp_backward_loops(X, A, B, n: int, dY):
    """Pure-Python version of tp_mlp_backward_full on nested lists: the same
    chain-rule steps, entry by entry.  Returns (dX, dA, dB) as nested lists."""
    X = [[float(v) for v in row] for row in X]
    A = [[float(v) for v in row] for row in A]
    B = [[float(v) for v in row] for row in B]
    dY = [[float(v) for v in row] for row in dY]
    D, F = len(A), len(A[0])
    M = len(X)
    if F % n:
        raise ValueError("F must be divisible by n")
    w = F // n
    dX = [[0.0] * D for _ in range(M)]
    dA = [[0.0] * F for _ in range(D)]
    dB = [[0.0] * D for _ in range(F)]
    for i in range(n):
        cols = range(i * w, (i + 1) * w)
        for f in cols:
            # column f of S = X A, of H = GeLU(S) and of dS
            s_col = [sum(X[m][d] * A[d][f] for d in range(D)) for m in range(M)]
            h_col = [gelu_scalar(v) for v in s_col]
            dh_col = [sum(dY[m][d] * B[f][d] for d in range(D)) for m in range(M)]
            ds_col = [dh_col[m] * gelu_grad_scalar(s_col[m]) for m in range(M)]
            for d in range(D):
                dB[f][d] = sum(h_col[m] * dY[m][d] for m in range(M))
                dA[d][f] = sum(X[m][d] * ds_col[m] for m in range(M))
        for m in range(M):
            for d in range(D):
                dX[m][d] += sum(
                    sum(dY[m][e] * B[f][e] for e in range(D))
                    * gelu_grad_scalar(sum(X[m][k] * A[k][f] for k in range(D))) * A[d][f]
                    for f in cols)
    return dX, dA, dB
