"""Parity at the largest sizes the C ABI accepts: each of M, D and F at 2^21
(the ABI's limit on a dimension), the others small, bf16; the backward
over 2^21 rows; and the attention half at its limits (one sequence of 2^21
tokens, and 65535 sequences).

These stress what only the largest shapes reach: the tile counts and grid
sizes of 2^21 rows or columns, the longest K loops (32768 steps of 64, with
an fp32 accumulator over 2^21 terms), and the 64-bit panel offsets of tiles
far into an operand.  The output and the workspace are filled with NaN first,
so a tile that writes nothing, or a read of H that was never written, fails;
the oracle checks one seeded row of every 256-row tile (rows of Y depend only
on the same rows of X), or every row where M is small.  One more row than the
limit is refused before any HIP call.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_transformer_mlp_tpmlp_amd as tp
from oracle import attention_oracle as ao
from parity_util import (assert_close, oracle_forward, sample_rows_per_tile, say, to_dev, to_f64,
                         workloads)

pytestmark = pytest.mark.gpu

MAX_DIM = 1 << 21
SHAPE = 2  # TPMLP_ERR_SHAPE


def _poisoned_forward(inp, n, **kw):
    dt = torch.bfloat16
    X, A, B = (to_dev(a, dt) for a in (inp.X, inp.A, inp.B))
    sh = tp.shard_mlp(A, B, n)
    M, D = X.shape
    flags = 1 if kw.get("layernorm") else 0  # TPMLP_OPT_LAYERNORM
    stream = torch.cuda.current_stream().cuda_stream
    ws = sh.workspace(tp.lib().tpmlp_forward_workspace_bytes(sh.handle, M, flags, 0), stream)
    ws.fill_(0xFF)  # NaN bit patterns everywhere in the workspace
    Y = torch.full((M, D), float("nan"), dtype=dt, device="cuda")
    if kw.pop("residual", False):
        kw["residual"] = X
    tp.tp_mlp(X, sh, out=Y, **kw)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Y).all()), "an element of Y was not written (or read a NaN)"
    return Y, sh, X


def test_max_rows():
    """M = 2^21 rows (D = 64, F = 128): 2^21 / 128 row tiles on both GEMMs,
    with and without the LayerNorm prologue and residual."""
    M, D, F, n = MAX_DIM, 64, 128, 2
    say(f"maximum M: M={M} D={D} F={F} n={n}")
    inp = workloads.random_case(M, D, F, seed=2101, dtype="bf16")
    rows = sample_rows_per_tile(M, 256, seed=2101)
    idx = torch.from_numpy(rows).cuda()
    Y, sh, X = _poisoned_forward(inp, n)
    assert_close(to_f64(Y[idx]), oracle_forward(inp.X[rows], inp.A, inp.B, n), "bf16", f"M=2^21, rows {len(rows)}")
    del Y
    Yl, _, _ = _poisoned_forward(inp, n, layernorm=True, residual=True)
    assert_close(to_f64(Yl[idx]), oracle_forward(inp.X[rows], inp.A, inp.B, n, layernorm=True, residual=True),
                 "bf16", f"M=2^21 LN+residual, rows {len(rows)}")
    del Yl
    L = tp.lib()
    assert L.tpmlp_forward_workspace_bytes(sh.handle, M + 1, 0, 0) == 0
    Yd = torch.empty((1, D), dtype=torch.bfloat16, device="cuda")
    assert L.tpmlp_forward_ex(X.data_ptr(), M + 1, sh.handle, Yd.data_ptr(), None, None) == SHAPE


def test_max_hidden():
    """D = 2^21 (M = 64, F = 64): GEMM1 runs a K loop of 2^21 / 64 = 32768
    steps into one fp32 accumulator; GEMM2 has 2^21 output columns."""
    M, D, F, n = 64, MAX_DIM, 64, 1
    say(f"maximum D: M={M} D={D} F={F} n={n}")
    inp = workloads.random_case(M, D, F, seed=2102, dtype="bf16")
    Y, _, _ = _poisoned_forward(inp, n)
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, n), "bf16", "D=2^21, every row")


def test_max_intermediate():
    """F = 2^21 over n = 2 shards (M = 64, D = 64): GEMM1 has 2^21 output
    columns, and GEMM2's K loop sums both shards' 2^20 columns each, 32768
    steps, in one fp32 accumulator."""
    M, D, F, n = 64, 64, MAX_DIM, 2
    say(f"maximum F: M={M} D={D} F={F} n={n}")
    inp = workloads.random_case(M, D, F, seed=2103, dtype="bf16")
    Y, _, _ = _poisoned_forward(inp, n)
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, n), "bf16", "F=2^21, every row")


def test_max_rows_backward():
    """The backward over M = 2^21 rows (D = 128, F = 256, n = 2).  dA and dB
    contract over the 2^21 rows: K-major K loops of 32768 steps, split into
    ranges because their two output tiles leave the GPU almost empty (fp32
    partials summed in range order)."""
    M, D, F, n = MAX_DIM, 128, 256, 2
    say(f"maximum M, backward: M={M} D={D} F={F} n={n}")
    inp = workloads.random_case(M, D, F, seed=2104, dtype="bf16")
    dY = workloads.round_to_bf16(np.random.default_rng(2105).standard_normal((M, D)).astype(np.float32))
    dt = torch.bfloat16
    X, A, B, tdY = (to_dev(a, dt) for a in (inp.X, inp.A, inp.B, dY))
    sh = tp.shard_mlp(A, B, n)
    dX, dA, dB = tp.tp_mlp_backward(X, tdY, sh)
    torch.cuda.synchronize()
    for t, name in ((dX, "dX"), (dA, "dA"), (dB, "dB")):
        assert bool(torch.isfinite(t).all()), f"{name} has a non-finite element"
    rX, rA, rB = oracle.tp_mlp_backward_full(inp.X, inp.A, inp.B, n, dY)
    assert_close(to_f64(dA), rA, "bf16", "dA over 2^21 rows")
    assert_close(to_f64(dB), rB, "bf16", "dB over 2^21 rows")
    assert_close(to_f64(dX), rX, "bf16", "dX, every row")


def _attn_weights(inp, heads, p):
    dt = torch.bfloat16
    x = to_dev(inp.x, dt)
    aw = tp.shard_attention(to_dev(inp.Wq, dt), to_dev(inp.Wk, dt), to_dev(inp.Wv, dt), heads, p)
    return x, aw


def test_attention_longest_sequence():
    """One sequence of 2^21 tokens (the token limit; one head of 64): every
    query row's softmax runs over 32768 key tiles.  Query rows are
    independent, so the oracle computes the sampled rows' attention over all
    2^21 keys and values."""
    seq, h = MAX_DIM, 64
    say(f"attention: one sequence of {seq} tokens, one head")
    inp = workloads.attn_case(1, seq, h, seed=2106)
    x, aw = _attn_weights(inp, 1, 1)
    out = tp.attention(x, 1, seq, aw, layernorm=False, residual=False)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rows = sample_rows_per_tile(seq, seq // 16, seed=2106)
    xs = inp.x.astype(np.float64)
    ref = ao.head_attention(xs[rows] @ inp.Wq, xs @ inp.Wk, xs @ inp.Wv)
    assert_close(to_f64(out[torch.from_numpy(rows).cuda()]), ref, "bf16", f"s=2^21, query rows {len(rows)}")


def test_attention_most_sequences():
    """65535 sequences (the batch limit, one grid dimension of the attention
    kernel) of 32 tokens; a sample of sequences against the oracle, each
    sequence on its own.  One more sequence is refused before any HIP call."""
    batch, seq, h = 65535, 32, 64
    say(f"attention: {batch} sequences of {seq} tokens, one head")
    inp = workloads.attn_case(batch, seq, h, seed=2107)
    x, aw = _attn_weights(inp, 1, 1)
    out = tp.attention(x, batch, seq, aw, layernorm=False, residual=False)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    seqs = sample_rows_per_tile(batch, 2048, seed=2107)
    got, ref = [], []
    for b in seqs:
        t = slice(b * seq, (b + 1) * seq)
        xb = inp.x[t].astype(np.float64)
        ref.append(ao.head_attention(xb @ inp.Wq, xb @ inp.Wk, xb @ inp.Wv))
        got.append(to_f64(out[b * seq:(b + 1) * seq]))
    assert_close(np.concatenate(got), np.concatenate(ref), "bf16", f"b=65535, sequences {len(seqs)}")
    L = tp.lib()
    assert L.tpmlp_attn_workspace_bytes(aw.handle, batch + 1, seq) == 0
    nbytes = L.tpmlp_attn_workspace_bytes(aw.handle, batch, seq)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    assert L.tpmlp_attention(x.data_ptr(), batch + 1, seq, aw.handle, out.data_ptr(), 0, 0.0, ws.data_ptr(),
                             nbytes, None, None) == SHAPE
