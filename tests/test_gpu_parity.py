"""GPU parity: the HIP path against the fp64 oracle, element by element.

Every call goes through the C ABI (the ctypes binding of include/tpmlp.h).
Small and mid sizes are compared on every output element; the full-size
workloads are compared on a seeded sample of rows (rows of Y depend only on
the same rows of X, so the oracle computes exactly those rows).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import tensor_transformer_mlp_tpmlp_amd as tp
from parity_util import (TOL_BF16, TOL_F32, assert_close, oracle_forward, sample_rows, sample_rows_per_tile,
                         say, to_dev, to_f64, torch_dtype)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tp.lib()
    yield
    torch.cuda.synchronize()


def _run(inp, n, dtype, **kw):
    dt = torch_dtype(dtype)
    X, A, B = to_dev(inp.X, dt), to_dev(inp.A, dt), to_dev(inp.B, dt)
    sh = tp.shard_mlp(A, B, n)
    if kw.pop("residual", False):
        kw["residual"] = X
    Y = tp.tp_mlp(X, sh, **kw)
    torch.cuda.synchronize()
    return Y, sh, (X, A, B)


# ---------------------------------------------------------------------------
# the worked example and the tiny fp32 workload
# ---------------------------------------------------------------------------

def test_worked_example_f32():
    say("worked example fp32 M=1 D=2 F=4 n=2")
    inp = workloads.worked_example()
    Y, sh, _ = _run(inp, 2, "f32")
    ref = oracle_forward(inp.X, inp.A, inp.B, 2)
    assert_close(to_f64(Y), ref, "f32", "worked example Y")
    assert np.all(np.abs(to_f64(Y) - np.array([[1.682, 2.796]])) <= 5e-4)
    _, parts = oracle.shard_outputs(inp.X, oracle.shard_mlp(inp.A, inp.B, 2))
    X = to_dev(inp.X, torch.float32)
    printed = [[[0.841, 1.955]], [[0.841, 0.841]]]
    for i in range(2):
        Yi = to_f64(tp.tp_mlp(X, sh, shard_index=i))
        assert_close(Yi, parts[i], "f32", f"worked example partial Y_{i}")
        assert np.all(np.abs(Yi - np.array(printed[i])) <= 5e-4)


def test_worked_example_bf16():
    say("worked example bf16")
    inp = workloads.worked_example()  # small integers: exact in bf16
    Y, _, _ = _run(inp, 2, "bf16", out_dtype=torch.float32)
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, 2), "bf16", "worked example bf16")


def test_tiny_f32_workload_and_partials():
    w = workloads.WORKLOADS["tiny_f32"]
    say(f"tiny fp32 workload {w.note}")
    inp = workloads.make_inputs(w)
    Y, sh, (X, _, _) = _run(inp, w.n, "f32")
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, w.n), "f32", "tiny_f32 Y")
    _, parts = oracle.shard_outputs(inp.X, oracle.shard_mlp(inp.A, inp.B, w.n))
    for i in range(w.n):
        Yi = to_f64(tp.tp_mlp(X, sh, shard_index=i))
        assert_close(Yi, parts[i], "f32", f"tiny_f32 partial Y_{i}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_invariance_every_divisor(dtype):
    """The result equals the unsplit one for every N dividing F."""
    w = workloads.WORKLOADS["tiny_f32"]
    inp = workloads.make_inputs(w)
    if dtype == "bf16":
        inp = workloads.Inputs(workloads.round_to_bf16(inp.X), workloads.round_to_bf16(inp.A),
                               workloads.round_to_bf16(inp.B))
    ref = oracle_forward(inp.X, inp.A, inp.B, 1)
    F = inp.A.shape[1]
    outs = {}
    for n in [d for d in range(1, F + 1) if F % d == 0]:
        say(f"split invariance {dtype} n={n}")
        Y, _, _ = _run(inp, n, dtype, out_dtype=torch.float32)
        outs[n] = to_f64(Y)
        assert_close(outs[n], ref, dtype, f"n={n}")


# ---------------------------------------------------------------------------
# shapes spanning several tiles, ragged tails, both kernel families
# ---------------------------------------------------------------------------

SHAPES = [
    # (M, D, F, n, dtype)
    (1, 2, 4, 2, "f32"),
    (3, 5, 7, 7, "f32"),
    (130, 70, 96, 3, "f32"),
    (200, 100, 330, 5, "f32"),
    (1, 64, 256, 4, "bf16"),
    (257, 129, 384, 4, "bf16"),
    (300, 256, 512, 2, "bf16"),
    (256, 64, 256, 1, "bf16"),
    (256, 128, 256, 1, "bf16"),     # GEMM1 K = 128: generic kernel; GEMM2 on 128x128 tiles
    (512, 256, 512, 2, "bf16"),     # 128x128 tiles, K = 256 and 512
    (512, 384, 1536, 4, "bf16"),
    (512, 256, 1024, 4, "bf16"),
    (768, 512, 768, 3, "bf16"),
    (1280, 768, 2560, 5, "bf16"),
]


@pytest.mark.parametrize("M,D,F,n,dtype", SHAPES)
def test_shapes(M, D, F, n, dtype):
    say(f"shape M={M} D={D} F={F} n={n} {dtype}")
    inp = workloads.random_case(M, D, F, seed=M * 7 + D * 3 + F + n, dtype=dtype)
    Y, _, _ = _run(inp, n, dtype)
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, n), dtype, f"M={M} D={D} F={F} n={n}")


# The throughput GEMM streams K (64-wide steps) through a ring of LDS units
# with its last step peeled.  For 256x256 tiles of row-major operands the
# loop body is written out for the five phases of the ring's slots and
# leaves after any of them, so these shapes run 1 to 7 steps on 256x256
# tiles (GEMM1 with M x F = 4096 x 4096, or GEMM2 with M x D = 4096 x 4096;
# the other GEMM is small and takes small tiles) and a short loop on 128x128.
RING_SHAPES = [
    # (M, D, F, n): which GEMM hits the ring with how many K steps
    (4096, 64, 4096, 1),    # GEMM1 256x256, 1 step (no loop)
    (4096, 128, 4096, 2),   # GEMM1 256x256, 2 steps
    (4096, 192, 4096, 1),   # GEMM1 256x256, 3 steps
    (4096, 256, 4096, 2),   # GEMM1 256x256, 4 steps
    (4096, 320, 4096, 4),   # GEMM1 256x256, 5 steps
    (4096, 384, 4096, 2),   # GEMM1 256x256, 6 steps (all five phases, then the exit)
    (4096, 448, 4096, 1),   # GEMM1 256x256, 7 steps (the phases wrap around)
    (4096, 4096, 64, 1),    # GEMM2 256x256, 1 step
    (4096, 4096, 128, 1),   # GEMM2 256x256, 2 steps
    (4096, 4096, 192, 1),   # GEMM2 256x256, 3 steps
    (4096, 4096, 448, 1),   # GEMM2 256x256, 7 steps
    (512, 192, 512, 2),     # GEMM1 128x128, 3 steps
    # The ten-slot tiles (64x64, 128x64) run one loop body over ten slots
    # (five steps of units, issued three steps ahead): short loops, and loops
    # longer than the ring, whose slot index wraps.
    (512, 64, 512, 1),      # GEMM1 64x64, 1 step; GEMM2 64x64, 8 steps
    (512, 128, 512, 1),     # GEMM1 64x64, 2 steps
    (512, 512, 64, 1),      # GEMM2 64x64, 1 step
    (512, 512, 192, 1),     # GEMM2 64x64, 3 steps
    (512, 512, 256, 2),     # GEMM2 64x64, 4 steps
    (512, 512, 320, 1),     # GEMM2 64x64, 5 steps
    (512, 512, 384, 2),     # GEMM2 64x64, 6 steps
    (512, 512, 704, 1),     # GEMM2 64x64, 11 steps
    (2048, 1024, 64, 1),    # GEMM2 128x64, 1 step; GEMM1 64x64, 16 steps
    (2048, 1024, 128, 2),   # GEMM2 128x64, 2 steps
    (2048, 1024, 192, 1),   # GEMM2 128x64, 3 steps
    (2048, 1024, 384, 2),   # GEMM2 128x64, 6 steps
    (2048, 1024, 704, 1),   # GEMM1 128x64, 16 steps; GEMM2 128x64, 11 steps
]


@pytest.mark.parametrize("M,D,F,n", RING_SHAPES)
def test_ring_short_k(M, D, F, n):
    say(f"short K ring M={M} D={D} F={F} n={n}")
    inp = workloads.random_case(M, D, F, seed=M + 3 * D + 5 * F + n, dtype="bf16")
    Y, _, _ = _run(inp, n, "bf16")
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, n), "bf16", f"M={M} D={D} F={F} n={n}")


def test_narrow_tiles_short_k_residual_fp32():
    """GEMM2 with few output tiles (M = D = 1024) and a short K loop
    (K = F = 768, 12 steps): it runs on narrow tiles with the whole K loop in
    one accumulator (the forward never splits the shard sum), with the
    residual and the fp32 cast in its epilogue."""
    M, D, F, n = 1024, 1024, 768, 2
    say(f"narrow tiles, short K, M={M} D={D} F={F} n={n} residual fp32")
    inp = workloads.random_case(M, D, F, seed=77, dtype="bf16")
    Y, _, _ = _run(inp, n, "bf16", residual=True, out_dtype=torch.float32)
    ref = oracle_forward(inp.X, inp.A, inp.B, n, residual=True)
    assert_close(to_f64(Y), ref, "bf16", "narrow tiles, residual, fp32 out")
    Yn, _, _ = _run(inp, n, "bf16")
    assert_close(to_f64(Yn), oracle_forward(inp.X, inp.A, inp.B, n), "bf16", "narrow tiles, bf16 out")


@pytest.mark.parametrize("M,D,F,n", [(512, 256, 1024, 4), (300, 96, 200, 2)])
def test_layernorm_residual_shapes(M, D, F, n):
    say(f"LN+residual M={M} D={D} F={F} n={n}")
    inp = workloads.random_case(M, D, F, seed=5 + M, dtype="bf16", sx=2.0)
    inp.X[:] = workloads.round_to_bf16(inp.X + 3.0)  # a non-zero row mean
    Y, _, _ = _run(inp, n, "bf16", layernorm=True, residual=True)
    ref = oracle_forward(inp.X, inp.A, inp.B, n, layernorm=True, residual=True)
    assert_close(to_f64(Y), ref, "bf16", "LN+residual out")
    Yn, _, _ = _run(inp, n, "bf16", layernorm=True)
    assert_close(to_f64(Yn), oracle_forward(inp.X, inp.A, inp.B, n, layernorm=True), "bf16", "LN, no residual")


@pytest.mark.parametrize("offset,spread", [(1024.0, 16.0), (8192.0, 16.0)])
def test_layernorm_large_row_mean(offset, spread):
    """Rows whose mean is large next to their spread (|mu| / sigma about 60
    and about 500 after the bf16 rounding of x): the LayerNorm prologue's
    correction r (x A - mu sum(A)) cancels most of x A, and the Norm after
    the residual normalises an fp32 sum with the same offset.  Both must
    still match the oracle, which normalises first, in fp64."""
    M, D, F, n = 512, 1024, 2048, 4
    say(f"LayerNorm, large row mean: offset {offset}, spread {spread}")
    inp = workloads.random_case(M, D, F, seed=int(offset), dtype="bf16", sx=spread)
    inp.X[:] = workloads.round_to_bf16(inp.X + np.float32(offset))
    xs = inp.X.astype(np.float64)
    say(f"row |mean| / std after rounding: {float(np.median(np.abs(xs.mean(1)) / xs.std(1))):.0f}")
    Y, _, _ = _run(inp, n, "bf16", layernorm=True, residual=True)
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, n, layernorm=True, residual=True), "bf16",
                 "LN first + residual")
    Yn, _, _ = _run(inp, n, "bf16", layernorm=True)
    assert_close(to_f64(Yn), oracle_forward(inp.X, inp.A, inp.B, n, layernorm=True), "bf16", "LN first")
    Ya, _, _ = _run(inp, n, "bf16", layernorm_after=True, residual=True)
    assert_close(to_f64(Ya), oracle_forward(inp.X, inp.A, inp.B, n, residual=True, layernorm_after=True), "bf16",
                 "Norm after the residual")


# ---------------------------------------------------------------------------
# the bf16 workloads at their full sizes
# ---------------------------------------------------------------------------

def test_workload_h1024_full():
    w = workloads.WORKLOADS["mlp_h1024_bf16"]
    say(f"{w.name}: {w.note}")
    inp = workloads.make_inputs(w)
    Y, _, _ = _run(inp, w.n, "bf16")
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, w.n), "bf16", w.name)


@pytest.mark.parametrize("name", ["mlp_h4096_bf16", "rank_h8192_bf16"])
def test_workload_large_sampled_rows(name):
    """The full-size workloads, with Y and the whole workspace (H) filled
    with NaN before the forward: every element of Y must then be finite
    (every output tile written, no stale H read), and one seeded row of
    every 256-row tile, plus the first and last rows, is compared with the
    oracle (rows of Y depend only on the same rows of X).  A second forward
    into a fresh NaN-filled output must give the same Y bit for bit (no
    race between tiles, at the size the bench times)."""
    w = workloads.WORKLOADS[name]
    say(f"{w.name}: {w.note} (NaN-poisoned Y and workspace, a row of every 256-row tile)")
    inp = workloads.make_inputs(w)
    dt = torch.bfloat16
    X, A, B = to_dev(inp.X, dt), to_dev(inp.A, dt), to_dev(inp.B, dt)
    sh = tp.shard_mlp(A, B, w.n)
    stream = torch.cuda.current_stream().cuda_stream
    ws = sh.workspace(tp.lib().tpmlp_forward_workspace_bytes(sh.handle, w.M, 0, 0), stream)
    ws.fill_(0xFF)  # NaN bit patterns everywhere in the workspace
    Y = torch.full((w.M, w.D), float("nan"), dtype=dt, device="cuda")
    tp.tp_mlp(X, sh, out=Y)
    Y2 = torch.full_like(Y, float("nan"))
    tp.tp_mlp(X, sh, out=Y2)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(Y).all()), "an element of Y was not written (or read a NaN)"
    assert torch.equal(Y, Y2), "two forwards on the same inputs differ"
    del Y2
    rows = sample_rows_per_tile(w.M, 256, seed=w.seed)
    assert len(rows) >= w.M // 256
    got = to_f64(Y[torch.from_numpy(rows).to(Y.device)])
    ref = oracle_forward(inp.X[rows], inp.A, inp.B, w.n)
    assert_close(got, ref, "bf16", f"{w.name} rows {len(rows)}")


def test_wide_output_residual_fp32_sampled_rows():
    """GEMM2 with 256 output tiles of 256x256 (N = D = 4096), a residual and
    fp32 output; GEMM1 (N = F = 2048) runs on 128x128 tiles."""
    M, D, F, n = 4096, 4096, 2048, 2
    say(f"wide output residual fp32 M={M} D={D} F={F} n={n}")
    inp = workloads.random_case(M, D, F, seed=21, dtype="bf16")
    Y, _, _ = _run(inp, n, "bf16", residual=True, out_dtype=torch.float32)
    rows = sample_rows(M, 24, seed=21)
    ref = oracle_forward(inp.X[rows], inp.A, inp.B, n, residual=True)
    got = to_f64(Y[torch.from_numpy(rows).to(Y.device)])
    assert_close(got, ref, "bf16", "wide output, residual, fp32 out")
    # the residual must not hide MLP errors: the same rows without it
    Yn, _, _ = _run(inp, n, "bf16", out_dtype=torch.float32)
    got = to_f64(Yn[torch.from_numpy(rows).to(Yn.device)])
    assert_close(got, oracle_forward(inp.X[rows], inp.A, inp.B, n), "bf16", "wide output, no residual")


@pytest.mark.parametrize("s", [128, 256, 512])
def test_workload_postln_full(s):
    w = workloads.WORKLOADS[f"postln_s{s}_bf16"]
    say(f"{w.name}: {w.note}")
    inp = workloads.make_inputs(w)
    out, sh, (X, _, _) = _run(inp, w.n, "bf16", layernorm=True, residual=True)
    ref_out = oracle_forward(inp.X, inp.A, inp.B, w.n, layernorm=True, residual=True)
    assert_close(to_f64(out), ref_out, "bf16", f"{w.name} out = x + Y")
    # the residual must not hide MLP errors: check Y alone too
    Y = tp.tp_mlp(X, sh, layernorm=True)
    ref_Y = oracle_forward(inp.X, inp.A, inp.B, w.n, layernorm=True)
    assert_close(to_f64(Y), ref_Y, "bf16", f"{w.name} Y")


# ---------------------------------------------------------------------------
# partials, packing, GeLU, determinism, edge cases, error paths
# ---------------------------------------------------------------------------

def test_shard_index_partials_bf16():
    say("partials bf16 M=512 D=256 F=1024 n=4")
    inp = workloads.random_case(512, 256, 1024, seed=77, dtype="bf16")
    Y, sh, (X, _, _) = _run(inp, 4, "bf16", out_dtype=torch.float32)
    _, parts = oracle.shard_outputs(inp.X, oracle.shard_mlp(inp.A, inp.B, 4))
    total = torch.zeros_like(Y)
    for i in range(4):
        Yi = tp.tp_mlp(X, sh, shard_index=i, out_dtype=torch.float32)
        assert_close(to_f64(Yi), parts[i], "bf16", f"partial Y_{i}")
        total += Yi
    assert_close(to_f64(total), to_f64(Y), "bf16", "sum of partials vs fused sum")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unpack_is_bit_exact(dtype):
    say(f"unpack {dtype}")
    inp = workloads.random_case(4, 96, 320, seed=9, dtype=dtype)
    dt = torch_dtype(dtype)
    A, B = to_dev(inp.A, dt), to_dev(inp.B, dt)
    for n in (1, 4, 5, 320):
        sh = tp.shard_mlp(A, B, n)
        w = 320 // n
        pairs = sh.pairs()
        torch.cuda.synchronize()
        assert len(pairs) == n
        for i, (A_i, B_i) in enumerate(pairs):
            assert torch.equal(A_i, A[:, i * w:(i + 1) * w])
            assert torch.equal(B_i, B[i * w:(i + 1) * w, :])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("count", [1, 7, 8, 9, 4099, (1 << 20) + 5])
def test_gelu_kernel(dtype, count):
    say(f"gelu {dtype} count={count}")
    rng = np.random.default_rng(count)
    x = (rng.standard_normal(count) * 3).astype(np.float32)
    x[:min(count, 4)] = np.array([0.0, 1.0, 2.0, -30.0], np.float32)[:min(count, 4)]
    dt = torch_dtype(dtype)
    xd = to_dev(x if dtype == "f32" else workloads.round_to_bf16(x), dt)
    y = tp.gelu(xd)
    ref = oracle.gelu(to_f64(xd))
    got = to_f64(y)
    if dtype == "f32":
        assert np.all(np.abs(got - ref) <= 2e-6 * np.maximum(np.abs(ref), 1e-3))
    else:  # one bf16 rounding of the result
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    if count >= 2:
        assert got[0] == 0.0
    tp.gelu(xd, out=xd)  # in place
    torch.cuda.synchronize()
    assert torch.equal(xd, y)


def test_determinism_and_every_tile_written():
    w = workloads.WORKLOADS["mlp_h1024_bf16"]
    say("determinism + NaN-poisoned outputs, mlp_h1024_bf16")
    inp = workloads.make_inputs(w)
    X, A, B = (to_dev(a, torch.bfloat16) for a in (inp.X, inp.A, inp.B))
    sh = tp.shard_mlp(A, B, w.n)
    y1 = torch.full((w.M, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    ws = sh.workspace(tp.lib().tpmlp_forward_workspace_bytes(sh.handle, w.M, 0, 0), stream)
    ws.fill_(0xFF)  # NaN bit patterns in H
    tp.tp_mlp(X, sh, out=y1)
    y2 = torch.full_like(y1, float("nan"))
    tp.tp_mlp(X, sh, out=y2)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y1).all())
    assert torch.equal(y1, y2)


def test_two_streams_at_once_share_no_workspace():
    """One descriptor used by forwards on two streams at the same time: the
    binding gives each stream its own workspace (H), so each result equals
    its sequential one bit for bit."""
    say("two streams, one descriptor, concurrent forwards")
    M, D, F, n = 1024, 512, 2048, 4
    inp1 = workloads.random_case(M, D, F, seed=91, dtype="bf16")
    inp2 = workloads.random_case(M, D, F, seed=92, dtype="bf16")
    dt = torch.bfloat16
    A, B = to_dev(inp1.A, dt), to_dev(inp1.B, dt)
    X1, X2 = to_dev(inp1.X, dt), to_dev(inp2.X, dt)
    sh = tp.shard_mlp(A, B, n)
    ref1, ref2 = tp.tp_mlp(X1, sh), tp.tp_mlp(X2, sh)
    Y1, Y2 = torch.empty_like(ref1), torch.empty_like(ref2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(8):
        with torch.cuda.stream(s1):
            tp.tp_mlp(X1, sh, out=Y1)
        with torch.cuda.stream(s2):
            tp.tp_mlp(X2, sh, out=Y2)
    torch.cuda.synchronize()
    assert torch.equal(Y1, ref1)
    assert torch.equal(Y2, ref2)


def test_empty_and_single_row():
    say("M=0 and M=1")
    inp = workloads.random_case(1, 256, 1024, seed=3, dtype="bf16")
    dt = torch.bfloat16
    X, A, B = to_dev(inp.X, dt), to_dev(inp.A, dt), to_dev(inp.B, dt)
    sh = tp.shard_mlp(A, B, 4)
    Y0 = tp.tp_mlp(X[:0], sh)
    assert Y0.shape == (0, 256)
    Y1 = tp.tp_mlp(X, sh)
    torch.cuda.synchronize()
    assert_close(to_f64(Y1), oracle_forward(inp.X, inp.A, inp.B, 4), "bf16", "M=1")


def test_layernorm_constant_rows_give_residual():
    say("LN of constant rows")
    inp = workloads.random_case(256, 256, 512, seed=4, dtype="bf16")
    inp.X[:] = 1.5
    out, _, (X, _, _) = _run(inp, 2, "bf16", layernorm=True, residual=True)
    assert torch.equal(out, X)  # LN(const) = 0, GeLU(0) = 0, so out = x exactly


def test_forward_errors_with_real_descriptor():
    say("error paths")
    inp = workloads.random_case(64, 64, 128, seed=2, dtype="f32")
    X, A, B = (to_dev(a, torch.float32) for a in (inp.X, inp.A, inp.B))
    sh = tp.shard_mlp(A, B, 2)
    L = tp.lib()
    Y = torch.empty(64, 64, device="cuda")
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    assert L.tpmlp_set_workspace(sh.handle, small.data_ptr(), small.numel()) == 0
    assert L.tpmlp_forward(X.data_ptr(), 64, sh.handle, Y.data_ptr(), None) == 5  # workspace too small
    assert L.tpmlp_forward(X.data_ptr(), -1, sh.handle, Y.data_ptr(), None) == 2
    assert L.tpmlp_forward(X.data_ptr() + 4, 64, sh.handle, Y.data_ptr(), None) == 6
    with pytest.raises(tp.TpmlpError):
        tp.tp_mlp(X, sh, shard_index=2)
    with pytest.raises(tp.TpmlpError):
        tp.tp_mlp(X, sh, out_dtype=torch.bfloat16)
    with pytest.raises(tp.TpmlpError):
        tp.shard_mlp(A, B[:, :], 3)
    big = torch.empty(L.tpmlp_forward_workspace_bytes(sh.handle, 64, 0, 0), dtype=torch.uint8, device="cuda")
    assert L.tpmlp_set_workspace(sh.handle, big.data_ptr(), big.numel()) == 0
    assert L.tpmlp_forward(X.data_ptr(), 64, sh.handle, Y.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert_close(to_f64(Y), oracle_forward(inp.X, inp.A, inp.B, 2), "f32", "tpmlp_forward with bound workspace")
    import ctypes
    d_, f_, n_, t_ = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int(), ctypes.c_int()
    assert L.tpmlp_shard_info(sh.handle, ctypes.byref(d_), ctypes.byref(f_), ctypes.byref(n_), ctypes.byref(t_)) == 0
    assert (d_.value, f_.value, n_.value, t_.value) == (64, 128, 2, 0)
    assert L.tpmlp_shard_count(sh.handle) == 2
    assert L.tpmlp_shard_unpack(sh.handle, 2, None, None, None) == 2
