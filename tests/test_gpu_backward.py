"""GPU parity of the backward pass (tpmlp_backward) against the fp64 oracle.

Every call goes through the C ABI.  Small and mid sizes are compared on every
element of dX, dA and dB.  The headline size is compared on samples that are
exactly the oracle of a sub-problem: rows of dX depend only on the same rows
of X and dY (the oracle of that sub-batch), and column f of dA / row f of dB
depend only on column f of A and row f of B (the oracle of the MLP restricted
to the sampled intermediate columns).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import tensor_transformer_mlp_tpmlp_amd as tp
from parity_util import assert_close, sample_rows, say, to_dev, to_f64, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tp.lib()
    yield
    torch.cuda.synchronize()


def _case(M, D, F, seed, dtype, sdy=1.0):
    inp = workloads.random_case(M, D, F, seed=seed, dtype=dtype)
    dY = np.random.default_rng(seed + 1).standard_normal((M, D)).astype(np.float32) * sdy
    if dtype == "bf16":
        dY = workloads.round_to_bf16(dY)
    return inp, dY


def _gpu_backward(inp, dY, n, dtype):
    dt = torch_dtype(dtype)
    X, A, B, tdY = (to_dev(a, dt) for a in (inp.X, inp.A, inp.B, dY))
    sh = tp.shard_mlp(A, B, n)
    dX, dA, dB = tp.tp_mlp_backward(X, tdY, sh)
    torch.cuda.synchronize()
    return dX, dA, dB


BWD_SHAPES = [
    # (M, D, F, n, dtype)
    (1, 2, 4, 2, "f32"),
    (3, 5, 7, 7, "f32"),
    (130, 70, 96, 3, "f32"),
    (60, 36, 100, 5, "f32"),        # multiples of 4: vector transposes, ragged tiles
    (64, 64, 256, 4, "bf16"),
    (257, 129, 384, 4, "bf16"),     # odd sizes: the bounds-checked kernel
    (200, 136, 264, 3, "bf16"),     # multiples of 8: vector transposes, ragged tiles
    (512, 256, 1024, 4, "bf16"),    # every GEMM on the 128x128 ring kernel
    (1024, 512, 2048, 2, "bf16"),
    (256, 4096, 3072, 3, "bf16"),   # weight gradients on 256x256 tiles, both operands K-major
]


@pytest.mark.parametrize("M,D,F,n,dtype", BWD_SHAPES)
def test_backward_shapes(M, D, F, n, dtype):
    say(f"backward M={M} D={D} F={F} n={n} {dtype}")
    inp, dY = _case(M, D, F, seed=900 + M + D + F + n, dtype=dtype)
    dX, dA, dB = _gpu_backward(inp, dY, n, dtype)
    rX, rA, rB = oracle.tp_mlp_backward_full(inp.X, inp.A, inp.B, n, dY)
    assert_close(to_f64(dX), rX, dtype, "dX")
    assert_close(to_f64(dA), rA, dtype, "dA")
    assert_close(to_f64(dB), rB, dtype, "dB")


def test_backward_h1024_full():
    w = workloads.WORKLOADS["mlp_h1024_bf16"]
    say(f"backward {w.name}")
    inp = workloads.make_inputs(w)
    dY = workloads.round_to_bf16(np.random.default_rng(w.seed + 7).standard_normal((w.M, w.D)).astype(np.float32))
    dX, dA, dB = _gpu_backward(inp, dY, w.n, "bf16")
    rX, rA, rB = oracle.tp_mlp_backward_full(inp.X, inp.A, inp.B, w.n, dY)
    assert_close(to_f64(dX), rX, "bf16", "dX")
    assert_close(to_f64(dA), rA, "bf16", "dA")
    assert_close(to_f64(dB), rB, "bf16", "dB")


def test_backward_headline_sampled():
    w = workloads.WORKLOADS["mlp_h4096_bf16"]
    say(f"backward {w.name} (twice; sampled rows of dX, columns of dA, rows of dB)")
    inp = workloads.make_inputs(w)
    dY = workloads.round_to_bf16(np.random.default_rng(w.seed + 7).standard_normal((w.M, w.D)).astype(np.float32))
    dX, dA, dB = _gpu_backward(inp, dY, w.n, "bf16")
    assert bool(torch.isfinite(dX).all()) and bool(torch.isfinite(dA).all()) and bool(torch.isfinite(dB).all())
    # a second backward on the same inputs gives the same gradients bit for bit
    again = _gpu_backward(inp, dY, w.n, "bf16")
    for x, y, name in zip((dX, dA, dB), again, ("dX", "dA", "dB")):
        assert torch.equal(x, y), f"two backwards differ in {name}"
    del again
    rows = sample_rows(w.M, 16, seed=w.seed)
    rX, _, _ = oracle.tp_mlp_backward_full(inp.X[rows], inp.A, inp.B, w.n, dY[rows])
    assert_close(to_f64(dX[torch.from_numpy(rows).to(dX.device)]), rX, "bf16", f"dX rows {len(rows)}")
    cols = sample_rows(w.F, 16, seed=w.seed + 1)
    _, rA, rB = oracle.tp_mlp_backward_full(inp.X, inp.A[:, cols], inp.B[cols, :], 1, dY)
    idx = torch.from_numpy(cols).to(dA.device)
    assert_close(to_f64(dA[:, idx]), rA, "bf16", f"dA columns {len(cols)}")
    assert_close(to_f64(dB[idx, :]), rB, "bf16", f"dB rows {len(cols)}")


def test_backward_empty_batch_gives_zero_weight_grads():
    say("backward M = 0")
    inp, dY = _case(4, 64, 128, seed=3, dtype="bf16")
    A, B = to_dev(inp.A, torch.bfloat16), to_dev(inp.B, torch.bfloat16)
    sh = tp.shard_mlp(A, B, 2)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    dX, dA, dB = tp.tp_mlp_backward(X, X.clone(), sh)
    torch.cuda.synchronize()
    assert dX.shape == (0, 64)
    assert float(dA.float().abs().max()) == 0.0 and float(dB.float().abs().max()) == 0.0
    # through the C ABI: an empty batch needs no workspace, so NULL is accepted
    L = tp.lib()
    assert L.tpmlp_backward_workspace_bytes(sh.handle, 0) == 0
    dA2 = torch.full((64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    dB2 = torch.full((128, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    assert L.tpmlp_backward(None, None, 0, sh.handle, None, None, None, dA2.data_ptr(), dB2.data_ptr(),
                            None, 0, None) == 0
    torch.cuda.synchronize()
    assert float(dA2.float().abs().max()) == 0.0 and float(dB2.float().abs().max()) == 0.0


def test_backward_deterministic():
    say("backward determinism")
    inp, dY = _case(512, 256, 1024, seed=5, dtype="bf16")
    a = _gpu_backward(inp, dY, 4, "bf16")
    b = _gpu_backward(inp, dY, 4, "bf16")
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_errors_with_real_descriptor():
    say("backward error paths")
    inp, dY = _case(64, 64, 128, seed=2, dtype="f32")
    X, A, B, tdY = (to_dev(a, torch.float32) for a in (inp.X, inp.A, inp.B, dY))
    sh = tp.shard_mlp(A, B, 2)
    L = tp.lib()
    dX = torch.empty_like(X)
    dA = torch.empty(64, 128, device="cuda")
    dB = torch.empty(128, 64, device="cuda")
    need = L.tpmlp_backward_workspace_bytes(sh.handle, 64)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    args = (X.data_ptr(), tdY.data_ptr(), 64, sh.handle, None, None, dX.data_ptr(), dA.data_ptr(), dB.data_ptr())
    assert L.tpmlp_backward(*args, ws.data_ptr(), need - 1, None) == 5      # workspace too small
    assert L.tpmlp_backward(*args, None, need, None) == 5
    assert L.tpmlp_backward(X.data_ptr(), tdY.data_ptr(), -1, sh.handle, None, None, dX.data_ptr(), dA.data_ptr(),
                            dB.data_ptr(), ws.data_ptr(), need, None) == 2
    assert L.tpmlp_backward(X.data_ptr() + 4, tdY.data_ptr(), 64, sh.handle, None, None, dX.data_ptr(),
                            dA.data_ptr(), dB.data_ptr(), ws.data_ptr(), need, None) == 6
    assert L.tpmlp_backward(X.data_ptr(), tdY.data_ptr(), 64, sh.handle, None, X.data_ptr() + 4, dX.data_ptr(),
                            dA.data_ptr(), dB.data_ptr(), ws.data_ptr(), need, None) == 6   # act misaligned
    assert L.tpmlp_backward(X.data_ptr(), tdY.data_ptr(), 64, sh.handle, None, None, dX.data_ptr(), None,
                            dB.data_ptr(), ws.data_ptr(), need, None) == 1
    assert L.tpmlp_backward(*args, ws.data_ptr(), need, None) == 0
    torch.cuda.synchronize()
    rX, rA, rB = oracle.tp_mlp_backward_full(inp.X, inp.A, inp.B, 2, dY)
    assert_close(to_f64(dX), rX, "f32", "dX")
    assert_close(to_f64(dA), rA, "f32", "dA")
    assert_close(to_f64(dB), rB, "f32", "dB")


@pytest.mark.parametrize("M,D,F,n,dtype", [(512, 256, 1024, 4, "bf16"), (130, 70, 96, 3, "f32")])
def test_forward_saves_preact_and_backward_uses_it(M, D, F, n, dtype):
    """save_preact returns S = X A (the oracle's, to the dtype's tolerance), and
    a backward given that S is bit-identical to one that recomputes it (the
    same GEMM produces both)."""
    say(f"save_preact M={M} D={D} F={F} n={n} {dtype}")
    inp, dY = _case(M, D, F, seed=4242 + M, dtype=dtype)
    dt = torch_dtype(dtype)
    X, A, B, tdY = (to_dev(a, dt) for a in (inp.X, inp.A, inp.B, dY))
    sh = tp.shard_mlp(A, B, n)
    S = torch.empty((M, F), dtype=dt, device="cuda")
    Y = tp.tp_mlp(X, sh, save_preact=S)
    torch.cuda.synchronize()
    assert_close(to_f64(S), inp.X.astype(np.float64) @ inp.A.astype(np.float64), dtype, "saved pre-activation")
    assert_close(to_f64(Y), oracle.tp_mlp(inp.X, oracle.shard_mlp(inp.A, inp.B, n)), dtype, "forward with save")
    with_s = tp.tp_mlp_backward(X, tdY, sh, preact=S)
    torch.cuda.synchronize()
    without = tp.tp_mlp_backward(X, tdY, sh)
    torch.cuda.synchronize()
    for a, b in zip(with_s, without):
        assert torch.equal(a, b)


@pytest.mark.parametrize("M,D,F,n,dtype", [(512, 256, 1024, 4, "bf16"), (1024, 512, 2048, 2, "bf16"),
                                           (130, 70, 96, 3, "f32")])
def test_backward_with_kept_activation(M, D, F, n, dtype):
    """A forward that keeps S (save_preact) and H (save_act): the kept H is
    GeLU of the oracle's S to the dtype's tolerance, the forward's Y is
    unchanged by keeping it, and a backward given both matches the oracle
    gradients.  Its dX and dA are bit-identical to those of the backward that
    recomputes H (they do not read H); dB uses the forward's H, which was
    rounded once from fp32 rather than from the rounded S."""
    say(f"save_act M={M} D={D} F={F} n={n} {dtype}")
    inp, dY = _case(M, D, F, seed=5151 + M, dtype=dtype)
    dt = torch_dtype(dtype)
    X, A, B, tdY = (to_dev(a, dt) for a in (inp.X, inp.A, inp.B, dY))
    sh = tp.shard_mlp(A, B, n)
    S = torch.full((M, F), float("nan"), dtype=dt, device="cuda")
    H = torch.full((M, F), float("nan"), dtype=dt, device="cuda")
    Y = tp.tp_mlp(X, sh, save_preact=S, save_act=H)
    Y0 = tp.tp_mlp(X, sh)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y0)
    s_ref = inp.X.astype(np.float64) @ inp.A.astype(np.float64)
    assert_close(to_f64(H), oracle.gelu(s_ref), dtype, "kept activation")
    kept = tp.tp_mlp_backward(X, tdY, sh, preact=S, act=H)
    torch.cuda.synchronize()
    rebuilt = tp.tp_mlp_backward(X, tdY, sh, preact=S)
    torch.cuda.synchronize()
    assert torch.equal(kept[0], rebuilt[0]) and torch.equal(kept[1], rebuilt[1])
    rX, rA, rB = oracle.tp_mlp_backward_full(inp.X, inp.A, inp.B, n, dY)
    for got, ref, nm in zip(kept, (rX, rA, rB), ("dX", "dA", "dB")):
        assert_close(to_f64(got), ref, dtype, nm + " (kept H)")


def test_kept_activation_of_one_shard_and_alignment():
    """save_act with shard_index = i receives GPU i's H_i (M x F/n), the same
    values as columns iF/n .. (i+1)F/n - 1 of the all-shards H; its partial
    Y_i is unchanged by keeping it; a misaligned save_act is TPMLP_ERR_ALIGN
    before any work."""
    import ctypes
    M, D, F, n = 512, 256, 1024, 4
    say(f"save_act with shard_index M={M} D={D} F={F} n={n}")
    inp, _ = _case(M, D, F, seed=6161, dtype="bf16")
    X, A, B = (to_dev(a, torch.bfloat16) for a in (inp.X, inp.A, inp.B))
    sh = tp.shard_mlp(A, B, n)
    H = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    tp.tp_mlp(X, sh, save_act=H)
    w = F // n
    for i in (0, n - 1):
        Hi = torch.full((M, w), float("nan"), dtype=torch.bfloat16, device="cuda")
        Yi = tp.tp_mlp(X, sh, shard_index=i, save_act=Hi)
        Yi0 = tp.tp_mlp(X, sh, shard_index=i)
        torch.cuda.synchronize()
        assert torch.equal(Hi, H[:, i * w:(i + 1) * w])
        assert torch.equal(Yi, Yi0)
    L = tp.lib()
    need = L.tpmlp_forward_workspace_bytes(sh.handle, M, 0, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    Y = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    o = tp.tpmlp.Opts()
    L.tpmlp_opts_init(ctypes.byref(o))
    o.workspace, o.workspace_bytes = ws.data_ptr(), ws.numel()
    o.save_act = H.data_ptr() + 4
    assert L.tpmlp_forward_ex(X.data_ptr(), M, sh.handle, Y.data_ptr(), ctypes.byref(o), None) == 6


def _colwise_err(got, ref, axis):
    """Largest normwise error over columns (axis 0) or rows (axis 1), each
    scaled by its own max |ref|: columns of very different magnitude are
    each checked at their own scale."""
    scale = np.max(np.abs(ref), axis=axis)
    err = np.max(np.abs(got - ref), axis=axis) / np.where(scale > 0, scale, 1.0)
    return float(np.max(err))


def test_gelu_saturation_forward_and_backward():
    """GeLU and its derivative far into both tails, through the fused
    epilogues: column j of A is scaled by 10^e_j, e_j cycling over -2 .. 29,
    so S = X A reaches about 1e30 in magnitude (x^2 overflows fp32 inside
    the GeLU, and the derivative's polynomial q overflows while s(1 - s) is
    exactly 0).  GeLU(s) must tend to s and to 0, GeLU'(s) to 1 and to 0,
    with no NaN; H is checked column by column and dB row by row at their
    own scale, against the fp64 oracle."""
    M, D, F, n = 128, 64, 256, 2
    say(f"GeLU saturation, forward and backward, |S| up to ~1e30, M={M} D={D} F={F} n={n}")
    inp, dY = _case(M, D, F, seed=4242, dtype="bf16")
    scale = 10.0 ** (np.arange(F) % 32 - 2)
    A = workloads.round_to_bf16((inp.A * scale[None, :]).astype(np.float32))
    assert np.all(np.isfinite(A))
    dt = torch.bfloat16
    X, tA, B, tdY = (to_dev(a, dt) for a in (inp.X, A, inp.B, dY))
    sh = tp.shard_mlp(tA, B, n)
    S = torch.empty((M, F), dtype=dt, device="cuda")
    H = torch.empty((M, F), dtype=dt, device="cuda")
    Y = tp.tp_mlp(X, sh, save_preact=S, save_act=H)
    Y0 = tp.tp_mlp(X, sh)  # the plain GeLU epilogue, keeping nothing
    dX, dA, dB = tp.tp_mlp_backward(X, tdY, sh, preact=S, act=H)
    dX2, dA2, dB2 = tp.tp_mlp_backward(X, tdY, sh)  # S and H recomputed
    torch.cuda.synchronize()
    assert torch.equal(Y, Y0)
    for t, name in ((S, "S"), (H, "H"), (Y, "Y"), (dX, "dX"), (dA, "dA"), (dB, "dB")):
        assert bool(torch.isfinite(t).all()), f"{name} has a non-finite element"
    S_ref = inp.X.astype(np.float64) @ A.astype(np.float64)
    assert float(np.max(np.abs(S_ref))) > 1e29
    err_h = _colwise_err(to_f64(H), oracle.gelu(S_ref), axis=0)
    say(f"H, column by column at its own scale: max error {err_h:.3e}")
    assert err_h <= 1e-2
    assert_close(to_f64(Y), oracle.tp_mlp(inp.X, oracle.shard_mlp(A, inp.B, n)), "bf16", "Y")
    rX, rA, rB = oracle.tp_mlp_backward_full(inp.X, A, inp.B, n, dY)
    assert_close(to_f64(dX), rX, "bf16", "dX")
    err_a = _colwise_err(to_f64(dA), rA, axis=0)
    err_b = _colwise_err(to_f64(dB), rB, axis=1)
    say(f"dA column by column: {err_a:.3e}; dB row by row: {err_b:.3e}")
    assert err_a <= 1e-2 and err_b <= 1e-2
    # dX and dA do not read H: the same bits with S and H recomputed; dB uses
    # the H recomputed from the rounded S, checked at its own scale
    assert torch.equal(dX, dX2) and torch.equal(dA, dA2)
    assert bool(torch.isfinite(dB2).all())
    assert _colwise_err(to_f64(dB2), rB, axis=1) <= 1e-2
