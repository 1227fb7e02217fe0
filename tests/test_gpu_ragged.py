"""GPU parity of ragged shapes on the throughput kernel: token counts and
output widths that are not whole tiles ("Tensor Parallelism in Megatron-LM",
section 9, on kernels meeting shapes they were not built for).

The bf16 GEMMs take M (rows) and N (output columns) of any size, with K a
whole number of 64-wide steps: edge tiles clamp their operand rows and store
only rows below M and columns below N.  Outputs and the workspace start as
NaN, so every element must be written and nothing unwritten may be read.
"""

import numpy as np
import pytest
import torch

import workloads
import tensor_transformer_mlp_tpmlp_amd as tp
from parity_util import assert_close, oracle_forward, sample_rows_per_tile, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tp.lib()
    yield
    torch.cuda.synchronize()


def _poisoned_forward(inp, n, **kw):
    bf = torch.bfloat16
    X, A, B = to_dev(inp.X, bf), to_dev(inp.A, bf), to_dev(inp.B, bf)
    sh = tp.shard_mlp(A, B, n)
    M, D = inp.X.shape
    flags = (tp.OPT_LAYERNORM if kw.get("layernorm") else 0)
    stream = torch.cuda.current_stream().cuda_stream
    ws = sh.workspace(tp.lib().tpmlp_forward_workspace_bytes(sh.handle, M, flags, 0), stream)
    ws.fill_(0xFF)
    Y = torch.full((M, D), float("nan"), dtype=kw.get("out_dtype") or bf, device="cuda")
    if kw.pop("residual", False):
        kw["residual"] = X
    tp.tp_mlp(X, sh, out=Y, **kw)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Y).all()), "an element of Y was not written"
    return Y


# (M, D, F, n): D and F multiples of 64 (K of both GEMMs whole steps) but not
# of 128, or N = D not even a multiple of 64 (GEMM1 then takes the generic
# path, GEMM2 the throughput kernel with a ragged N), ragged M everywhere.
RAGGED = [
    (1, 128, 256, 2),
    (17, 192, 320, 5),
    (255, 256, 512, 2),
    (257, 1088, 4160, 4),
    (513, 1000, 2048, 4),
    (1000, 1088, 4160, 4),
    (2047, 1024, 4096, 4),
    (4000, 1024, 4096, 4),
    (4100, 2112, 4224, 3),
]


@pytest.mark.parametrize("M,D,F,n", RAGGED)
def test_ragged_shapes(M, D, F, n):
    say(f"ragged M={M} D={D} F={F} n={n}")
    inp = workloads.random_case(M, D, F, seed=M + D + F + n, dtype="bf16")
    Y = _poisoned_forward(inp, n)
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, n), "bf16", f"M={M} D={D} F={F} n={n}")


@pytest.mark.parametrize("M,D,F,n", [(1000, 1088, 4160, 4), (300, 1024, 4096, 4)])
def test_ragged_layernorm_residual_fp32(M, D, F, n):
    say(f"ragged LN + residual, fp32 out, M={M} D={D} F={F} n={n}")
    inp = workloads.random_case(M, D, F, seed=7 * M + n, dtype="bf16", sx=2.0)
    inp.X[:] = workloads.round_to_bf16(inp.X + 1.5)
    Y = _poisoned_forward(inp, n, layernorm=True, residual=True, out_dtype=torch.float32)
    ref = oracle_forward(inp.X, inp.A, inp.B, n, layernorm=True, residual=True)
    assert_close(to_f64(Y), ref, "bf16", "ragged LN + residual")
    Yn = _poisoned_forward(inp, n, layernorm=True)
    assert_close(to_f64(Yn), oracle_forward(inp.X, inp.A, inp.B, n, layernorm=True), "bf16",
                 "ragged LN, no residual")


def test_ragged_headline_m16383():
    """The headline sizes with one token fewer (M = 16383): the last row of
    256x256 tiles is one row short."""
    w = workloads.WORKLOADS["mlp_h4096_bf16"]
    M = w.M - 1
    say(f"headline shape with M={M}")
    inp = workloads.make_inputs(w)
    inp = workloads.Inputs(inp.X[:M].copy(), inp.A, inp.B)
    Y = _poisoned_forward(inp, w.n)
    rows = sample_rows_per_tile(M, 256, seed=M)
    ref = oracle_forward(inp.X[rows], inp.A, inp.B, w.n)
    assert_close(to_f64(Y[torch.from_numpy(rows).to(Y.device)]), ref, "bf16", f"M={M}, {len(rows)} rows")


def test_partial_and_full_agree_on_shared_rows():
    """A forward over the first M' rows gives bit-identical rows to the
    forward over all M rows (rows are independent; a ragged edge tile
    computes its rows exactly as an interior tile would)."""
    M, D, F, n = 2048, 1024, 4096, 4
    say(f"row prefixes agree bit for bit, M={M} D={D} F={F}")
    inp = workloads.random_case(M, D, F, seed=99, dtype="bf16")
    bf = torch.bfloat16
    X, A, B = to_dev(inp.X, bf), to_dev(inp.A, bf), to_dev(inp.B, bf)
    sh = tp.shard_mlp(A, B, n)
    full = tp.tp_mlp(X, sh)
    for Mp in (1, 100, 1000, 2047):
        part = tp.tp_mlp(X[:Mp].contiguous(), sh)
        torch.cuda.synchronize()
        assert torch.equal(part, full[:Mp]), f"M'={Mp}"
