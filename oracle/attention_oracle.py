"""fp64 CPU oracle for the attention half of the Megatron block (head-sharded
self-attention).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes (sources: "Tensor Parallelism in Megatron" section 4
"Attention: Split Heads", and the code walkthrough of "LLM Lab Notes 06:
Building a Megatron-Style Transformer Block from Scratch", section 2,
markers 2 to 4):

  * x_n = LayerNorm(x) over the hidden axis, no affine (marker 2; optional);
  * rank i of p owns H/p consecutive heads; for each of its heads,
    Q = x_n W^Q, K = x_n W^K, V = x_n W^V restricted to that head's d
    columns, and O = softmax(Q K^T / sqrt(d)) V over the tokens of one
    sequence (section 4, the local-attention equation); no mask;
  * the ranks' outputs are either concatenated along the hidden axis in rank
    order (marker 3: all_gather then cat, no output projection) or passed
    through the row-parallel output projection and summed over ranks
    (section 4: the output projection is row-parallel and reduces);
  * the residual x is added once (marker 4).

Readings (where the pages are silent or disagree):
  * The walkthrough's code multiplies q and k after a view to
    (batch, seq, heads, d) without moving the head axis forward, which taken
    literally would mix heads at each position rather than tokens.  The
    equation of section 4 and the walkthrough's own timing remark (attention
    cost growing with the square of the sequence) fix attention over the
    tokens of each sequence, per head; that is what is computed here.
  * Head j owns columns j*d .. (j+1)*d - 1 of W^Q, W^K, W^V (the view to
    (heads, d) in the code), and rank i owns heads i*H/p .. (i+1)*H/p - 1.
  * The softmax is the plain one, evaluated with the row maximum subtracted
    first (the same function, without overflow).

Everything is float64 numpy in the order stated; a pure-Python version
(``*_loops``) exists for tiny inputs.  Every function is pinned by
``tests/test_oracle_attention.py``.
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .tpmlp_oracle import layer_norm, layer_norm_loops, LN_EPS


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def softmax(z, axis: int = -1) -> np.ndarray:
    """exp(z) / sum(exp(z)) along `axis`, with the maximum subtracted first."""
    z = _f64(z)
    e = np.exp(z - np.max(z, axis=axis, keepdims=True))
    return e / np.sum(e, axis=axis, keepdims=True)


def head_attention(Q, K, V) -> np.ndarray:
    """O = softmax(Q K^T / sqrt(d)) V for one head of one sequence.

    "Tensor Parallelism in Megatron", section 4, the local-attention
    equation.  Q: (s_q, d), K: (s_k, d), V: (s_k, d_v); no mask.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    d = Q.shape[-1]
    return softmax((Q @ K.T) / math.sqrt(d), axis=-1) @ V


def head_columns(j: int, d: int) -> slice:
    """Columns of W^Q, W^K, W^V (and rows of W^O) that belong to head j."""
    return slice(j * d, (j + 1) * d)


def rank_heads(i: int, H: int, p: int) -> range:
    """Heads owned by rank i of p: H/p consecutive heads (section 4)."""
    if p <= 0 or H % p:
        raise ValueError("the number of heads must be divisible by the TP size")
    lh = H // p
    return range(i * lh, (i + 1) * lh)


def rank_attention(xn, Wq, Wk, Wv, H: int, p: int, i: int, batch: int, seq: int) -> np.ndarray:
    """O_i: rank i's heads for every sequence, (batch*seq, (H/p)*d).

    xn holds batch*seq token rows, sequence b in rows b*seq .. (b+1)*seq-1.
    """
    xn = _f64(xn)
    h = xn.shape[1]
    d = h // H
    heads = rank_heads(i, H, p)
    out = np.zeros((batch * seq, len(heads) * d))
    for t, j in enumerate(heads):
        c = head_columns(j, d)
        for b in range(batch):
            rows = slice(b * seq, (b + 1) * seq)
            x_b = xn[rows]
            Q = x_b @ _f64(Wq)[:, c]
            K = x_b @ _f64(Wk)[:, c]
            V = x_b @ _f64(Wv)[:, c]
            out[rows, t * d:(t + 1) * d] = head_attention(Q, K, V)
    return out


def attention_half(x, Wq, Wk, Wv, H: int, p: int, batch: int, seq: int, Wo=None,
                   layernorm: bool = True, residual: bool = True, eps: float = LN_EPS) -> np.ndarray:
    """The attention half of the block on batch*seq token rows of width h.

    "LLM Lab Notes 06" section 2, markers 2 to 4, with the attention of
    "Tensor Parallelism in Megatron" section 4.  With Wo None the ranks'
    outputs are concatenated in rank order (marker 3); otherwise
    attn = sum_i O_i W^O_i with W^O_i the rows of W^O for rank i's heads
    (section 4, row-parallel output projection), summed in ascending i.
    """
    x = _f64(x)
    h = x.shape[1]
    if h % H:
        raise ValueError("the hidden size must be divisible by the number of heads")
    if x.shape[0] != batch * seq:
        raise ValueError("x must hold batch*seq rows")
    xn = layer_norm(x, eps) if layernorm else x
    outs = [rank_attention(xn, Wq, Wk, Wv, H, p, i, batch, seq) for i in range(p)]
    if Wo is None:
        attn = np.concatenate(outs, axis=1)
    else:
        Wo = _f64(Wo)
        w = h // p
        attn = np.zeros_like(x)
        for i, O_i in enumerate(outs):
            attn = attn + O_i @ Wo[i * w:(i + 1) * w, :]
    return x + attn if residual else attn


# ---------------------------------------------------------------------------
# pure-Python versions for tiny inputs
# ---------------------------------------------------------------------------

def softmax_loops(row: Sequence[float]) -> List[float]:
    m = max(row)
    e = [math.exp(v - m) for v in row]
    t = sum(e)
    return [v / t for v in e]


def _mat(A, B):
    return [[sum(a * B[k][j] for k, a in enumerate(r)) for j in range(len(B[0]))] for r in A]


def attention_half_loops(x, Wq, Wk, Wv, H: int, p: int, batch: int, seq: int, Wo=None,
                         layernorm: bool = True, residual: bool = True, eps: float = LN_EPS):
    """Pure-Python attention_half on nested lists: the same steps entry by entry."""
    x = [[float(v) for v in r] for r in x]
    h = len(x[0])
    d = h // H
    xn = layer_norm_loops(x, eps) if layernorm else x
    Qf, Kf, Vf = _mat(xn, Wq), _mat(xn, Wk), _mat(xn, Wv)
    cat = [[0.0] * h for _ in x]
    for j in range(H):
        for b in range(batch):
            for qi in range(seq):
                q = Qf[b * seq + qi][j * d:(j + 1) * d]
                scores = [sum(q[t] * Kf[b * seq + ki][j * d + t] for t in range(d)) / math.sqrt(d)
                          for ki in range(seq)]
                w = softmax_loops(scores)
                for t in range(d):
                    cat[b * seq + qi][j * d + t] = sum(w[ki] * Vf[b * seq + ki][j * d + t] for ki in range(seq))
    if Wo is None:
        attn = cat
    else:
        # row-parallel: rank i contributes its heads' columns times its rows of W^O
        w = h // p
        attn = [[0.0] * h for _ in x]
        for i in range(p):
            part = _mat([r[i * w:(i + 1) * w] for r in cat], [list(map(float, r)) for r in Wo[i * w:(i + 1) * w]])
            attn = [[a + c for a, c in zip(ra, rc)] for ra, rc in zip(attn, part)]
    if residual:
        return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(x, attn)]
    return attn
