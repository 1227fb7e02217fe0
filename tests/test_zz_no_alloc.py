"""tpmlp_forward_noalloc: the forward with the library's own scratch array
as its workspace, for callers that cannot allocate.  Through the C ABI, its
output must equal tpmlp_forward_ex's (same kernels, a caller-owned
workspace) bit for bit and match the oracle, on two calls in a row, the
second with a smaller input; sizes beyond the array are rejected before any
HIP call, and the calls take no device memory."""

import ctypes

import numpy as np
import pytest
import torch

import workloads
import tensor_transformer_mlp_tpmlp_amd as tp
from tensor_transformer_mlp_tpmlp_amd import tpmlp as binding
from parity_util import assert_close, oracle_forward, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


def _free_bytes() -> int:
    hip = ctypes.CDLL("libamdhip64.so")
    free, total = ctypes.c_size_t(), ctypes.c_size_t()
    assert hip.hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
    return free.value


def _opts(flags=0, residual=None):
    o = binding.Opts()
    tp.lib().tpmlp_opts_init(ctypes.byref(o))
    o.flags = flags
    if residual is not None:
        o.residual = residual.data_ptr()
    return o


def test_noalloc_matches_forward_ex_twice_smaller_second():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L = tp.lib()
    w = workloads.WORKLOADS["postln_s256_bf16"]
    say(f"no-alloc forward: {w.name} then its first 512 rows, LayerNorm + residual")
    inp = workloads.make_inputs(w)
    bf = torch.bfloat16
    X, A, B = to_dev(inp.X, bf), to_dev(inp.A, bf), to_dev(inp.B, bf)
    sh = tp.shard_mlp(A, B, w.n)
    stream = torch.cuda.current_stream().cuda_stream
    flags = tp.OPT_LAYERNORM
    cases = [(w.M, X), (512, X[:512].contiguous())]
    # reference outputs through tpmlp_forward_ex with a caller-owned workspace
    refs = []
    for M, Xm in cases:
        assert L.tpmlp_forward_workspace_bytes(sh.handle, M, flags, 0) <= SCRATCH
        refs.append(tp.tp_mlp(Xm, sh, layernorm=True, residual=Xm))
    outs = [torch.full((M, w.D), float("nan"), dtype=bf, device="cuda") for M, _ in cases]
    torch.cuda.synchronize()
    # The first call on a device looks up the scratch array's address, which
    # loads the code object holding it (the array's one-time placement, kept
    # until the process ends); from then on a call takes no device memory.
    free = []
    for (M, Xm), Y in zip(cases, outs):
        o = _opts(flags, residual=Xm)
        st = L.tpmlp_forward_noalloc(Xm.data_ptr(), M, sh.handle, Y.data_ptr(), ctypes.byref(o), stream)
        assert st == 0, L.tpmlp_status_string(st)
        torch.cuda.synchronize()
        free.append(_free_bytes())
    say(f"device free memory after the first and the second no-alloc call: {free[0]} / {free[1]}")
    assert free[1] >= free[0], "the second no-alloc call took device memory"
    for (M, Xm), Y, R in zip(cases, outs, refs):
        assert torch.equal(Y, R), f"M={M}: no-alloc output differs from tpmlp_forward_ex"
        ref = oracle_forward(inp.X[:M], inp.A, inp.B, w.n, layernorm=True, residual=True)
        assert_close(to_f64(Y), ref, "bf16", f"no-alloc M={M}")
    # the plain MLP (no options, NULL opts) on the smaller input, once more
    Xs = cases[1][1]
    Y = torch.empty(512, w.D, dtype=bf, device="cuda")
    assert L.tpmlp_forward_noalloc(Xs.data_ptr(), 512, sh.handle, Y.data_ptr(), None, stream) == 0
    ref = tp.tp_mlp(Xs, sh)
    torch.cuda.synchronize()
    assert torch.equal(Y, ref)


def test_noalloc_rejects_what_does_not_fit():
    L = tp.lib()
    say("no-alloc forward: sizes beyond the scratch array, a caller workspace")
    inp = workloads.random_case(64, 1024, 4096, seed=5, dtype="bf16")
    bf = torch.bfloat16
    X, A, B = to_dev(inp.X, bf), to_dev(inp.A, bf), to_dev(inp.B, bf)
    sh = tp.shard_mlp(A, B, 4)
    Y = torch.empty(64, 1024, dtype=bf, device="cuda")
    big = 16384  # H alone is 128 MiB
    assert L.tpmlp_forward_workspace_bytes(sh.handle, big, 0, 0) > SCRATCH
    # rejected on the sizes alone, before any pointer is touched
    assert L.tpmlp_forward_noalloc(X.data_ptr(), big, sh.handle, Y.data_ptr(), None, None) == 5
    o = _opts()
    o.workspace = Y.data_ptr()
    o.workspace_bytes = Y.numel() * 2
    assert L.tpmlp_forward_noalloc(X.data_ptr(), 64, sh.handle, Y.data_ptr(), ctypes.byref(o), None) == 5
    assert L.tpmlp_forward_noalloc(X.data_ptr(), -1, sh.handle, Y.data_ptr(), None, None) == 2
    assert L.tpmlp_forward_noalloc(X.data_ptr(), 64, None, Y.data_ptr(), None, None) == 1
    assert L.tpmlp_forward_noalloc(X.data_ptr(), 0, sh.handle, Y.data_ptr(), None, None) == 0
    assert L.tpmlp_forward_noalloc(X.data_ptr(), 64, sh.handle, Y.data_ptr(), None, None) == 0
    torch.cuda.synchronize()
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, 4), "bf16", "no-alloc M=64")
