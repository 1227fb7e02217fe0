"""GPU parity of the LayerNorm-after placement, out = LayerNorm(x + TP-MLP(x)),
against the fp64 oracle (``oracle.norm_after_ffn``), through the C ABI.

Shapes cover both forms of the row-LayerNorm kernels: rows held in registers
(length a multiple of the 16-byte chunk, up to 64 x 8 chunks) and the
element-wise form (odd lengths, longer rows); the Post-LN workloads of
"LLM Lab Notes 06" are compared on every element.
"""

import ctypes

import numpy as np
import pytest
import torch

import workloads
import tensor_transformer_mlp_tpmlp_amd as tp
from parity_util import assert_close, oracle_forward, say, to_dev, to_f64, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tp.lib()
    yield
    torch.cuda.synchronize()


def _run(inp, n, dtype, residual=True, **kw):
    dt = torch_dtype(dtype)
    X, A, B = to_dev(inp.X, dt), to_dev(inp.A, dt), to_dev(inp.B, dt)
    sh = tp.shard_mlp(A, B, n)
    out = tp.tp_mlp(X, sh, residual=X if residual else None, **kw)
    torch.cuda.synchronize()
    return out, sh, X


AFTER_SHAPES = [
    # (M, D, F, n, dtype, residual)
    (1, 2, 4, 2, "f32", True),          # D % 4 != 0: element-wise Norm
    (37, 40, 96, 3, "f32", True),       # fp32 rows in registers, one chunk per lane
    (300, 96, 200, 2, "bf16", True),
    (257, 130, 384, 4, "bf16", True),   # odd D: element-wise Norm
    (512, 256, 1024, 4, "bf16", True),
    (512, 256, 1024, 4, "bf16", False),  # no residual: LayerNorm(Y)
    (64, 2048, 512, 2, "bf16", True),   # 8 chunks per lane, the longest register row
    (64, 2052, 256, 1, "bf16", True),   # one chunk longer: element-wise Norm
]


@pytest.mark.parametrize("M,D,F,n,dtype,residual", AFTER_SHAPES)
def test_norm_after_shapes(M, D, F, n, dtype, residual):
    say(f"LN after M={M} D={D} F={F} n={n} {dtype} residual={residual}")
    inp = workloads.random_case(M, D, F, seed=31 + M + D, dtype=dtype)
    out, _, _ = _run(inp, n, dtype, residual=residual, layernorm_after=True)
    ref = oracle_forward(inp.X, inp.A, inp.B, n, residual=residual, layernorm_after=True)
    assert_close(to_f64(out), ref, dtype, "LayerNorm(x + Y)" if residual else "LayerNorm(Y)")


def test_norm_after_fp32_output_and_eps():
    say("LN after, fp32 output, eps 1e-3")
    inp = workloads.random_case(512, 256, 1024, seed=8, dtype="bf16")
    out, _, _ = _run(inp, 4, "bf16", layernorm_after=True, out_dtype=torch.float32, eps=1e-3)
    ref = oracle_forward(inp.X, inp.A, inp.B, 4, residual=True, layernorm_after=True, eps=1e-3)
    assert out.dtype == torch.float32
    assert_close(to_f64(out), ref, "bf16", "LayerNorm(x + Y), fp32 out")


@pytest.mark.parametrize("s", [128, 256, 512])
def test_norm_after_postln_workloads_full(s):
    w = workloads.WORKLOADS[f"postln_s{s}_bf16"]
    say(f"{w.name} with the LayerNorm after: M={w.M} D={w.D} F={w.F} n={w.n}")
    inp = workloads.make_inputs(w)
    out, sh, X = _run(inp, w.n, "bf16", layernorm_after=True)
    ref = oracle_forward(inp.X, inp.A, inp.B, w.n, residual=True, layernorm_after=True)
    assert_close(to_f64(out), ref, "bf16", f"{w.name} LayerNorm(x + Y)")
    # every row normalised
    o = to_f64(out)
    assert np.max(np.abs(o.mean(axis=1))) < 2e-2
    assert np.max(np.abs(o.var(axis=1) - 1.0)) < 2e-2
    # bit-identical on a second call
    out2 = tp.tp_mlp(X, sh, residual=X, layernorm_after=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_layernorm_before_elementwise_stats():
    """The Norm-first placement with a row length that takes the element-wise
    statistics kernel (D not a multiple of 8)."""
    say("LN before, D=130")
    inp = workloads.random_case(200, 130, 256, seed=9, dtype="bf16", sx=2.0)
    inp.X[:] = workloads.round_to_bf16(inp.X + 3.0)
    out, _, _ = _run(inp, 2, "bf16", layernorm=True)
    ref = oracle_forward(inp.X, inp.A, inp.B, 2, layernorm=True, residual=True)
    assert_close(to_f64(out), ref, "bf16", "x + Y(LayerNorm(x)), element-wise statistics")


def test_norm_after_errors_and_workspace():
    say("LN after: error paths and workspace size")
    inp = workloads.random_case(64, 64, 128, seed=2, dtype="bf16")
    X, A, B = (to_dev(a, torch.bfloat16) for a in (inp.X, inp.A, inp.B))
    sh = tp.shard_mlp(A, B, 2)
    L = tp.lib()
    base = L.tpmlp_forward_workspace_bytes(sh.handle, 64, 0, 0)
    after = L.tpmlp_forward_workspace_bytes(sh.handle, 64, tp.OPT_LAYERNORM_AFTER, 0)
    assert after == base + 64 * 64 * 4
    ws = torch.empty(after, dtype=torch.uint8, device="cuda")
    Y = torch.empty(64, 64, dtype=torch.bfloat16, device="cuda")
    o = tp.tpmlp.Opts()
    L.tpmlp_opts_init(ctypes.byref(o))
    o.workspace, o.workspace_bytes = ws.data_ptr(), ws.numel()
    for flags, shard in ((3, -1), (2, 0), (4, -1)):
        o.flags, o.shard_index = flags, shard
        assert L.tpmlp_forward_ex(X.data_ptr(), 64, sh.handle, Y.data_ptr(), ctypes.byref(o), None) == 2
    o.flags, o.shard_index = tp.OPT_LAYERNORM_AFTER, -1
    o.workspace_bytes = after - 1
    assert L.tpmlp_forward_ex(X.data_ptr(), 64, sh.handle, Y.data_ptr(), ctypes.byref(o), None) == 5
    o.workspace_bytes = after
    assert L.tpmlp_forward_ex(X.data_ptr(), 64, sh.handle, Y.data_ptr(), ctypes.byref(o), None) == 0
    torch.cuda.synchronize()
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, 2, layernorm_after=True), "bf16",
                 "LayerNorm(Y) through tpmlp_forward_ex")
