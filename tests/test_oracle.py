"""Pins for the fp64 oracle (CPU only).

The oracle is the yardstick for every GPU parity test, so it is itself
checked against things it cannot agree with by construction:

* the values "Tensor-Parallel MLP (Megatron)" prints for its worked example
  (tests/golden/p4_worked_example.json) and its GeLU point values;
* the exact erf-GeLU (math.erf) that the tanh form approximates, and
  PyTorch's own tanh-GeLU and LayerNorm as library special cases;
* closed forms (GeLU(x) - GeLU(-x) = x; LayerNorm row mean 0, variance
  var/(var+eps));
* invariants the pages fix: the split result equals the unsplit result for
  every N dividing F ("Requirements"), plus permutation, scaling, zero and
  row-independence properties;
* an independent pure-Python implementation.

Each pin is a function of the implementation under test, and
``test_pins_reject_planted_mistakes`` feeds deliberately broken copies of the
oracle to the pins to show that plausible mistakes are caught.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p4_worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _close_to_print(got, printed, half_ulp):
    got = np.asarray(got, dtype=np.float64)
    printed = np.asarray(printed, dtype=np.float64)
    assert got.shape == printed.shape, (got.shape, printed.shape)
    return bool(np.all(np.abs(got - printed) <= half_ulp))


# ---------------------------------------------------------------------------
# pins, parameterised by the implementation they check
# ---------------------------------------------------------------------------

def pin_worked_example(gelu_fn, shard_fn, outputs_fn, tp_fn):
    g = _golden()
    X, A, B, n = np.array(g["X"], float), np.array(g["A"], float), np.array(g["B"], float), g["N"]
    p, h = g["printed"], g["half_ulp_of_print"]
    ok = True
    ok &= bool(np.array_equal(X @ A, np.array(p["XA"], float)))
    ok &= _close_to_print(gelu_fn(X @ A), p["H"], h)
    shards = shard_fn(A, B, n)
    ok &= len(shards) == 2
    Hs, Ys = outputs_fn(X, shards)
    ok &= _close_to_print(Hs[0], p["H0"], h) and _close_to_print(Hs[1], p["H1"], h)
    ok &= _close_to_print(Ys[0], p["Y0"], h) and _close_to_print(Ys[1], p["Y1"], h)
    Y = tp_fn(X, shards)
    ok &= _close_to_print(Y, p["Y"], h)
    ok &= _close_to_print(Ys[0] + Ys[1], p["Y0_plus_Y1"], h)
    return ok


def pin_gelu_points(gelu_fn):
    g = _golden()["gelu_points"]
    h = _golden()["half_ulp_of_print"]
    ok = float(gelu_fn(np.array(0.0))) == 0.0
    ok &= abs(float(gelu_fn(np.array(1.0))) - g["gelu_1"]) <= h
    ok &= abs(float(gelu_fn(np.array(2.0))) - g["gelu_2"]) <= h
    ok &= abs(2 * float(gelu_fn(np.array(1.0))) - g["gelu_1_plus_gelu_1"]) <= h
    return bool(ok)


def pin_gelu_vs_erf(gelu_fn):
    """The tanh form stays within 5e-4 of x*Phi(x) (exact GeLU) everywhere; its
    largest deviation is about 4.7e-4 near |x| ~ 2.  Also the Taylor terms at
    0 shared by both forms: slope 1/2 and curvature sqrt(2/pi)."""
    xs = np.linspace(-8.0, 8.0, 16001)
    exact = np.array([0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0))) for x in xs])
    ok = float(np.max(np.abs(gelu_fn(xs) - exact))) <= 5e-4
    e = 1e-4
    g = lambda v: float(gelu_fn(np.array(v)))
    ok &= abs((g(e) - g(-e)) / (2 * e) - 0.5) <= 1e-7
    ok &= abs((g(e) - 2 * g(0.0) + g(-e)) / (e * e) - math.sqrt(2.0 / math.pi)) <= 1e-4
    return bool(ok)


def pin_gelu_odd_identity(gelu_fn):
    """tanh is odd, so GeLU(x) - GeLU(-x) = x exactly in real arithmetic."""
    xs = np.linspace(-30.0, 30.0, 6001)
    return bool(np.all(np.abs(gelu_fn(xs) - gelu_fn(-xs) - xs) <= 1e-14 * np.maximum(1.0, np.abs(xs))))


def pin_gelu_vs_torch(gelu_fn):
    """PyTorch's tanh-approximate GeLU is a separate implementation of the same formula."""
    xs = np.linspace(-12.0, 12.0, 4801)
    ref = torch.nn.functional.gelu(torch.from_numpy(xs), approximate="tanh").numpy()
    return bool(np.max(np.abs(gelu_fn(xs) - ref)) <= 1e-14)


def pin_shard_ranges(shard_fn):
    """Pair i holds columns iF/n..(i+1)F/n-1 of A and the same rows of B, in order."""
    D, F = 3, 12
    A = np.array([[100 * f + d for f in range(F)] for d in range(D)], float)  # A[d, f] encodes f
    B = np.array([[100 * f + d for d in range(D)] for f in range(F)], float)  # B[f, d] encodes f
    ok = True
    for n in (1, 2, 3, 4, 6, 12):
        shards = shard_fn(A, B, n)
        ok &= len(shards) == n
        w = F // n
        for i, (A_i, B_i) in enumerate(shards):
            ok &= A_i.shape == (D, w) and B_i.shape == (w, D)
            cols = (A_i[0, :] // 100).astype(int).tolist()
            rows = (B_i[:, 0] // 100).astype(int).tolist()
            ok &= cols == list(range(i * w, (i + 1) * w)) and rows == cols
    return bool(ok)


def pin_split_invariance(shard_fn, tp_fn):
    """'The result must equal the unsplit GeLU(XA) B' for every divisor N of F."""
    inp = workloads.make_inputs(workloads.WORKLOADS["tiny_f32"])
    X, A, B = inp.X.astype(float), inp.A.astype(float), inp.B.astype(float)
    F = A.shape[1]
    ref = tp_fn(X, shard_fn(A, B, 1))
    scale = np.max(np.abs(ref))
    ok = True
    for n in [d for d in range(1, F + 1) if F % d == 0]:
        Y = tp_fn(X, shard_fn(A, B, n))
        ok &= float(np.max(np.abs(Y - ref))) <= 1e-12 * scale
    return bool(ok)


def pin_unsplit_is_torch_mlp(shard_fn, tp_fn):
    """N = 1 is the plain MLP; PyTorch's tanh-GeLU and matmul give it independently."""
    inp = workloads.make_inputs(workloads.WORKLOADS["tiny_f32"])
    X, A, B = (torch.from_numpy(a.astype(np.float64)) for a in (inp.X, inp.A, inp.B))
    ref = (torch.nn.functional.gelu(X @ A, approximate="tanh") @ B).numpy()
    ok = True
    for n in (1, 2, 8):
        Y = tp_fn(X.numpy(), shard_fn(A.numpy(), B.numpy(), n))
        ok &= float(np.max(np.abs(Y - ref))) <= 1e-12 * float(np.max(np.abs(ref)))
    return bool(ok)


def pin_layer_norm(ln_fn):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((9, 64)) * 3.0 + rng.standard_normal((9, 1)) * 5.0
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (64,)).numpy()
    y = ln_fn(x)
    ok = float(np.max(np.abs(y - ref))) <= 1e-12
    var = x.var(axis=1)
    ok &= bool(np.all(np.abs(y.mean(axis=1)) <= 1e-12))
    ok &= bool(np.all(np.abs(y.var(axis=1) - var / (var + oracle.LN_EPS)) <= 1e-12))
    return bool(ok)


def pin_post_ln(post_fn, shard_fn):
    """Residual is the un-normalised x, added once after the shard sum."""
    inp = workloads.random_case(6, 32, 64, seed=11)
    x, A, B = inp.X.astype(float), inp.A.astype(float), inp.B.astype(float)
    zeroB = np.zeros_like(B)
    ok = bool(np.array_equal(post_fn(x, shard_fn(A, zeroB, 4)), x))
    y1 = post_fn(x, shard_fn(A, B, 1))
    y4 = post_fn(x, shard_fn(A, B, 4))
    ok &= float(np.max(np.abs(y1 - y4))) <= 1e-12 * float(np.max(np.abs(y1)))
    # the FFN part sees LayerNorm(x): with torch's layer_norm and tanh-GeLU as the reference
    xt = torch.from_numpy(x)
    ffn = torch.nn.functional.gelu(torch.nn.functional.layer_norm(xt, (32,)) @ torch.from_numpy(A),
                                   approximate="tanh") @ torch.from_numpy(B)
    ok &= float(np.max(np.abs(y4 - (x + ffn.numpy())))) <= 1e-12 * float(np.max(np.abs(y4)))
    return bool(ok)


def pin_norm_after(after_fn, shard_fn):
    """out = LayerNorm(x + TP-MLP(x)): the FFN sees the raw x, the residual
    joins the shard sum, and the Norm comes last."""
    inp = workloads.random_case(6, 32, 64, seed=12)
    x, A, B = inp.X.astype(float), inp.A.astype(float) * 4.0, inp.B.astype(float) * 4.0
    xt = torch.from_numpy(x)
    F = torch.nn.functional
    # B = 0 reduces to the library LayerNorm of x
    ln_x = F.layer_norm(xt, (32,)).numpy()
    ok = float(np.max(np.abs(after_fn(x, shard_fn(A, np.zeros_like(B), 4)) - ln_x))) <= 1e-12
    # the whole composition with torch's layer_norm and tanh-GeLU
    ref = F.layer_norm(xt + F.gelu(xt @ torch.from_numpy(A), approximate="tanh") @ torch.from_numpy(B),
                       (32,)).numpy()
    y4 = after_fn(x, shard_fn(A, B, 4))
    ok &= float(np.max(np.abs(y4 - ref))) <= 1e-12
    # any split gives the same result
    ok &= float(np.max(np.abs(after_fn(x, shard_fn(A, B, 1)) - y4))) <= 1e-12
    # every row normalised: mean 0, biased variance v / (v + eps) of the pre-Norm row
    z = x + (F.gelu(xt @ torch.from_numpy(A), approximate="tanh") @ torch.from_numpy(B)).numpy()
    v = z.var(axis=1)
    ok &= bool(np.all(np.abs(y4.mean(axis=1)) <= 1e-12))
    ok &= bool(np.all(np.abs(y4.var(axis=1) - v / (v + oracle.LN_EPS)) <= 1e-12))
    return bool(ok)


# ---------------------------------------------------------------------------
# the oracle passes every pin
# ---------------------------------------------------------------------------

def test_worked_example_numpy():
    assert pin_worked_example(oracle.gelu, oracle.shard_mlp, oracle.shard_outputs, oracle.tp_mlp)


def test_worked_example_loops():
    g = _golden()
    Y, parts = oracle.tp_mlp_loops(g["X"], g["A"], g["B"], g["N"])
    h = g["half_ulp_of_print"]
    assert _close_to_print(Y, g["printed"]["Y"], h)
    assert _close_to_print(parts[0], g["printed"]["Y0"], h)
    assert _close_to_print(parts[1], g["printed"]["Y1"], h)


def test_gelu_points():
    assert pin_gelu_points(oracle.gelu)
    assert pin_gelu_points(np.vectorize(oracle.gelu_scalar))


def test_gelu_vs_exact_erf_form():
    assert pin_gelu_vs_erf(oracle.gelu)


def test_gelu_odd_identity():
    assert pin_gelu_odd_identity(oracle.gelu)


def test_gelu_vs_torch_tanh_gelu():
    assert pin_gelu_vs_torch(oracle.gelu)


def test_gelu_limits_and_nan():
    big = np.array([20.0, 50.0, 1e3, 1e30])
    assert np.all(oracle.gelu(big) == big)
    assert np.all(np.abs(oracle.gelu(-big)) <= 1e-80)
    assert np.isnan(oracle.gelu(np.array(np.nan)))


def test_shard_ranges():
    assert pin_shard_ranges(oracle.shard_mlp)


@pytest.mark.parametrize("n", [0, -1, 3, 5, 257])
def test_shard_rejects_bad_n(n):
    A = np.zeros((4, 256))
    B = np.zeros((256, 4))
    with pytest.raises(ValueError):
        oracle.shard_mlp(A, B, n)


def test_split_invariance_all_divisors():
    assert pin_split_invariance(oracle.shard_mlp, oracle.tp_mlp)


def test_unsplit_matches_torch_mlp():
    assert pin_unsplit_is_torch_mlp(oracle.shard_mlp, oracle.tp_mlp)


def test_loops_agree_with_numpy_tiny_workload():
    w = workloads.WORKLOADS["tiny_f32"]
    inp = workloads.make_inputs(w)
    Y, parts = oracle.tp_mlp_loops(inp.X.tolist(), inp.A.tolist(), inp.B.tolist(), w.n)
    shards = oracle.shard_mlp(inp.A, inp.B, w.n)
    ref = oracle.tp_mlp(inp.X, shards)
    _, ref_parts = oracle.shard_outputs(inp.X, shards)
    scale = np.max(np.abs(ref))
    assert np.max(np.abs(np.array(Y) - ref)) <= 1e-12 * scale
    for p, rp in zip(parts, ref_parts):
        assert np.max(np.abs(np.array(p) - rp)) <= 1e-12 * scale


def test_invariants():
    inp = workloads.random_case(5, 16, 48, seed=3)
    X, A, B = inp.X.astype(float), inp.A.astype(float), inp.B.astype(float)
    Y = oracle.tp_mlp(X, oracle.shard_mlp(A, B, 4))
    s = np.max(np.abs(Y))
    # permuting A's columns together with B's rows leaves the sum unchanged
    perm = np.random.default_rng(0).permutation(48)
    Yp = oracle.tp_mlp(X, oracle.shard_mlp(A[:, perm], B[perm, :], 4))
    assert np.max(np.abs(Yp - Y)) <= 1e-12 * s
    # Y is linear in B
    Y3 = oracle.tp_mlp(X, oracle.shard_mlp(A, -2.5 * B, 4))
    assert np.max(np.abs(Y3 + 2.5 * Y)) <= 1e-12 * s
    # zero input gives zero output (GeLU(0) = 0)
    assert np.all(oracle.tp_mlp(np.zeros_like(X), oracle.shard_mlp(A, B, 4)) == 0)
    # a zero column block of A zeroes exactly that shard's partial
    A0 = A.copy()
    A0[:, 12:24] = 0
    _, parts = oracle.shard_outputs(X, oracle.shard_mlp(A0, B, 4))
    assert np.all(parts[1] == 0) and np.any(parts[0] != 0)
    # rows are independent
    rows = [4, 0, 2]
    Yr = oracle.tp_mlp(X[rows], oracle.shard_mlp(A, B, 4))
    assert np.max(np.abs(Yr - Y[rows])) <= 1e-12 * s


def test_layer_norm():
    assert pin_layer_norm(oracle.layer_norm)
    x = np.random.default_rng(1).standard_normal((3, 10))
    assert np.max(np.abs(np.array(oracle.layer_norm_loops(x.tolist())) - oracle.layer_norm(x))) <= 1e-13
    # a constant row normalises to zero (variance 0, eps keeps it finite)
    assert np.all(oracle.layer_norm(np.full((2, 8), 3.25)) == 0)


def test_post_ln_block():
    assert pin_post_ln(oracle.post_ln_ffn, oracle.shard_mlp)


def test_norm_after_block():
    assert pin_norm_after(oracle.norm_after_ffn, oracle.shard_mlp)
    inp = workloads.random_case(3, 8, 12, seed=5)
    x, A, B = inp.X.astype(float), inp.A.astype(float), inp.B.astype(float)
    loops = np.array(oracle.norm_after_ffn_loops(x.tolist(), A.tolist(), B.tolist(), 3))
    assert np.max(np.abs(loops - oracle.norm_after_ffn(x, oracle.shard_mlp(A, B, 3)))) <= 1e-13
    # the two placements are different functions
    sh = oracle.shard_mlp(A, B, 3)
    assert np.max(np.abs(oracle.norm_after_ffn(x, sh) - oracle.post_ln_ffn(x, sh))) > 0.1


# ---------------------------------------------------------------------------
# planted mistakes must be caught by at least one pin
# ---------------------------------------------------------------------------

def _gelu_with(c=oracle.SQRT_2_OVER_PI, a=oracle.GELU_CUBIC, half=0.5, sign=1.0):
    def g(x):
        x = np.asarray(x, dtype=np.float64)
        return half * x * (1.0 + sign * np.tanh(c * (x + a * x ** 3)))
    return g


def _outputs_with(gelu_fn, transpose_b=False):
    def f(X, shards):
        Hs, Ys = [], []
        for A_i, B_i in shards:
            H = gelu_fn(np.asarray(X, float) @ A_i)
            Hs.append(H)
            Ys.append(H @ (B_i.T if transpose_b else B_i))
        return Hs, Ys
    return f


def _tp_with(outputs_fn, drop_last=False, residual_per_shard=False):
    def f(X, shards):
        _, Ys = outputs_fn(X, shards)
        if drop_last:
            Ys = Ys[:-1]
        return sum(Ys)
    return f


def _shard_with(offset=0, interleave=False):
    def f(A, B, n):
        A, B = np.asarray(A, float), np.asarray(B, float)
        F = A.shape[1]
        if F % n:
            raise ValueError
        w = F // n
        if interleave:
            return [(A[:, i::n], B[i::n, :]) for i in range(n)]
        out = []
        for i in range(n):
            lo = (i * w + offset) % F
            idx = [(lo + j) % F for j in range(w)]
            out.append((A[:, idx], B[idx, :]))
        return out
    return f


def test_pins_reject_planted_mistakes():
    good_g = oracle.gelu
    good_out = _outputs_with(good_g)
    good_tp = _tp_with(good_out)
    # the hand-made copies pass when unbroken
    assert pin_worked_example(good_g, oracle.shard_mlp, good_out, good_tp)
    assert pin_gelu_vs_erf(_gelu_with())

    bad_gelus = {
        "cubic 0.04715": _gelu_with(a=0.04715),
        "sqrt(pi/2)": _gelu_with(c=math.sqrt(math.pi / 2)),
        "no half": _gelu_with(half=1.0),
        "minus tanh": _gelu_with(sign=-1.0),
        "x instead of x^3": lambda x: 0.5 * np.asarray(x, float) * (1 + np.tanh(
            oracle.SQRT_2_OVER_PI * (np.asarray(x, float) * (1 + oracle.GELU_CUBIC)))),
        "erf form": lambda x: np.vectorize(lambda v: 0.5 * v * (1 + math.erf(v / math.sqrt(2))))(x),
    }
    for name, g in bad_gelus.items():
        caught = not (pin_gelu_points(g) and pin_gelu_vs_erf(g) and pin_gelu_vs_torch(g)
                      and pin_worked_example(g, oracle.shard_mlp, _outputs_with(g), _tp_with(_outputs_with(g))))
        assert caught, name

    # a dropped shard, a transposed B_i, or mis-sliced shards
    drop = _tp_with(good_out, drop_last=True)
    assert not (pin_worked_example(good_g, oracle.shard_mlp, good_out, drop)
                and pin_split_invariance(oracle.shard_mlp, drop))
    tb = _outputs_with(good_g, transpose_b=True)
    try:
        caught = not pin_worked_example(good_g, oracle.shard_mlp, tb, _tp_with(tb))
    except ValueError:
        caught = True
    assert caught
    assert not pin_shard_ranges(_shard_with(offset=1))
    assert not pin_shard_ranges(_shard_with(interleave=True))
    assert not pin_worked_example(good_g, _shard_with(interleave=True), good_out, good_tp)

    # LayerNorm: unbiased variance, missing eps, no centring
    def ln_unbiased(x):
        x = np.asarray(x, float)
        mu = x.mean(-1, keepdims=True)
        return (x - mu) / np.sqrt(x.var(-1, ddof=1, keepdims=True) + oracle.LN_EPS)

    def ln_no_eps(x):
        x = np.asarray(x, float)
        mu = x.mean(-1, keepdims=True)
        return (x - mu) / np.sqrt(x.var(-1, keepdims=True))

    def ln_no_centre(x):
        x = np.asarray(x, float)
        return x / np.sqrt(x.var(-1, keepdims=True) + oracle.LN_EPS)

    for bad in (ln_unbiased, ln_no_eps, ln_no_centre):
        assert not pin_layer_norm(bad), bad.__name__

    # Post-LN: residual of the normalised input, or added once per shard
    def post_normed_residual(x, shards):
        xn = oracle.layer_norm(x)
        return xn + oracle.tp_mlp(xn, shards)

    def post_per_shard(x, shards):
        xn = oracle.layer_norm(x)
        _, Ys = oracle.shard_outputs(xn, shards)
        return sum(np.asarray(x, float) + Y for Y in Ys)

    for bad in (post_normed_residual, post_per_shard):
        assert not pin_post_ln(bad, oracle.shard_mlp), bad.__name__

    # Norm after the residual: normalising first, no residual, the residual
    # outside the Norm, or the Norm taken per shard before the sum
    def after_norm_first(x, shards):
        return oracle.post_ln_ffn(x, shards)

    def after_no_residual(x, shards):
        return oracle.layer_norm(oracle.tp_mlp(x, shards))

    def after_residual_outside(x, shards):
        return np.asarray(x, float) + oracle.layer_norm(oracle.tp_mlp(x, shards))

    def after_per_shard(x, shards):
        _, Ys = oracle.shard_outputs(x, shards)
        return sum(oracle.layer_norm(np.asarray(x, float) + Y) for Y in Ys) / len(Ys)

    assert pin_norm_after(lambda x, sh: oracle.layer_norm(np.asarray(x, float) + oracle.tp_mlp(x, sh)),
                          oracle.shard_mlp)
    for bad in (after_norm_first, after_no_residual, after_residual_outside, after_per_shard):
        assert not pin_norm_after(bad, oracle.shard_mlp), bad.__name__
