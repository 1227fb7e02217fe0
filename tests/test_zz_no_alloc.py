"""tpmlp_forward_noalloc: the forward with the library's own scratch array
as its workspace, for callers that cannot allocate.  Through the C ABI, its
output must equal tpmlp_forward_ex's (same kernels, a caller-owned
workspace) bit for bit and match the oracle, on two calls in a row, the
second with a smaller input; sizes beyond the array are rejected before any
HIP call, and the calls take no device memory.  A graph captured around
the entry point replays it correctly on new inputs."""

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
REPLAYS = 3


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


def test_noalloc_forward_replays_from_a_captured_graph():
    """tpmlp_forward_noalloc under stream capture: the forward records kernel
    launches only (no allocation, no memset, no synchronising call), so a
    graph captured around it replays the same kernels on whatever the input
    buffers hold at replay time.  Two calls share one graph (Pre-LN with the
    residual, and the Norm-after placement, both on the scratch array); each
    replay follows an eager refill of the inputs and a synchronisation, and
    its outputs must equal tpmlp_forward_ex's on the same inputs bit for
    bit, and match the oracle on the last one."""
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L = tp.lib()
    w1 = workloads.WORKLOADS["postln_s128_bf16"]
    w2 = workloads.WORKLOADS["lnafter_s128_bf16"]
    say(f"captured no-alloc forward: {w1.name} then {w2.name}, {REPLAYS} replays")
    bf = torch.bfloat16
    inp = workloads.make_inputs(w1)
    sh = tp.shard_mlp(to_dev(inp.A, bf), to_dev(inp.B, bf), w1.n)
    M, D = w1.M, w1.D
    X1 = torch.empty(M, D, dtype=bf, device="cuda")
    X2 = torch.empty(M, D, dtype=bf, device="cuda")
    Y1 = torch.empty(M, D, dtype=bf, device="cuda")
    Y2 = torch.empty(M, D, dtype=bf, device="cuda")
    o1 = _opts(tp.OPT_LAYERNORM, X1)
    o2 = _opts(tp.OPT_LAYERNORM_AFTER, X2)
    # new inputs for every replay (and one for the warm-up), drawn on the host
    rng = np.random.default_rng(4242)
    draws = [(rng.standard_normal((M, D)), rng.standard_normal((M, D))) for _ in range(REPLAYS + 1)]

    def fill(k):
        X1.copy_(to_dev(draws[k][0], bf))
        X2.copy_(to_dev(draws[k][1], bf))

    def forward(stream):
        for X, Y, o in ((X1, Y1, o1), (X2, Y2, o2)):
            st = L.tpmlp_forward_noalloc(X.data_ptr(), M, sh.handle, Y.data_ptr(), ctypes.byref(o), stream)
            assert st == 0, L.tpmlp_status_string(st)

    # warm-up outside the capture: the first call on a device looks up the
    # scratch array's address, which is not a stream operation
    fill(REPLAYS)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        forward(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forward(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    for k in range(REPLAYS):
        fill(k)
        Y1.fill_(float("nan"))
        Y2.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # eager references on the same inputs through tpmlp_forward_ex
        R1 = tp.tp_mlp(X1, sh, layernorm=True, residual=X1)
        R2 = tp.tp_mlp(X2, sh, layernorm_after=True, residual=X2)
        torch.cuda.synchronize()
        say(f"replay {k}: comparing with the eager forward")
        assert torch.equal(Y1, R1), f"replay {k}: Pre-LN output differs from the eager forward"
        assert torch.equal(Y2, R2), f"replay {k}: Norm-after output differs from the eager forward"
    xs1 = to_f64(X1)
    xs2 = to_f64(X2)
    assert_close(to_f64(Y1), oracle_forward(xs1, inp.A, inp.B, w1.n, layernorm=True, residual=True),
                 "bf16", "captured Pre-LN")
    assert_close(to_f64(Y2), oracle_forward(xs2, inp.A, inp.B, w2.n, residual=True, layernorm_after=True),
                 "bf16", "captured Norm-after")
    del g
