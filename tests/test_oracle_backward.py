"""Pins of the oracle's backward pass (CPU only).

The backward is not printed on the pages, so the oracle's gradients are pinned
to what fixes them mathematically: central finite differences of the pinned
forward oracle, PyTorch autograd of the same expression in float64, the
derivative's limits, and the invariance of the gradients to the number of
shards.  A planted-mistake test checks that a dropped term, a skipped shard or
a swapped operand in the backward fails at least one pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# pins (each returns True when the implementation passes)
# ---------------------------------------------------------------------------

def pin_gelu_grad_fd(grad_fn):
    """Central differences of the pinned forward GeLU."""
    x = np.concatenate([np.linspace(-8, 8, 161), [-0.3, 1e-3, 2.5]])
    h = 1e-5
    fd = (oracle.gelu(x + h) - oracle.gelu(x - h)) / (2 * h)
    return bool(np.max(np.abs(grad_fn(x) - fd)) < 1e-8)


def pin_gelu_grad_limits(grad_fn):
    """g'(0) = 1/2 exactly; g' -> 1 for large x and -> 0 for very negative x."""
    g = grad_fn(np.array([0.0, 40.0, -40.0]))
    return bool(g[0] == 0.5 and abs(g[1] - 1.0) < 1e-12 and abs(g[2]) < 1e-12)


def pin_gelu_grad_torch(grad_fn):
    """PyTorch autograd of F.gelu(approximate='tanh') in float64."""
    x = torch.linspace(-6, 6, 97, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(x, approximate="tanh").sum().backward()
    return bool(np.max(np.abs(grad_fn(x.detach().numpy()) - x.grad.numpy())) < 1e-12)


def _tiny():
    M, D, F, n = 3, 4, 6, 2
    X = _rand((M, D), 1)
    A = _rand((D, F), 2, 0.5)
    B = _rand((F, D), 3, 0.5)
    dY = _rand((M, D), 4)
    return X, A, B, n, dY


def pin_backward_fd(back_fn):
    """Finite differences of L = sum(dY * Y(X, A, B)) with the pinned forward
    oracle, for every entry of X, A and B."""
    X, A, B, n, dY = _tiny()

    def loss(X_, A_, B_):
        return float(np.sum(dY * oracle.tp_mlp(X_, oracle.shard_mlp(A_, B_, n))))

    h = 1e-6
    grads = []
    for which, T in enumerate((X, A, B)):
        G = np.zeros_like(T)
        for idx in np.ndindex(T.shape):
            args_p = [X.copy(), A.copy(), B.copy()]
            args_m = [X.copy(), A.copy(), B.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            G[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        grads.append(G)
    dX, dA, dB = back_fn(X, A, B, n, dY)
    return all(np.max(np.abs(np.asarray(got) - ref)) < 1e-6 * max(1.0, np.max(np.abs(ref)))
               for got, ref in zip((dX, dA, dB), grads))


def pin_backward_torch(back_fn):
    """PyTorch autograd (float64) of sum_i gelu_tanh(X A_i) B_i."""
    M, D, F, n = 5, 8, 12, 3
    X, A, B, dY = _rand((M, D), 11), _rand((D, F), 12, 0.3), _rand((F, D), 13, 0.3), _rand((M, D), 14)
    tX, tA, tB = (torch.tensor(v, requires_grad=True) for v in (X, A, B))
    w = F // n
    Y = sum(torch.nn.functional.gelu(tX @ tA[:, i * w:(i + 1) * w], approximate="tanh") @ tB[i * w:(i + 1) * w]
            for i in range(n))
    Y.backward(torch.tensor(dY))
    got = back_fn(X, A, B, n, dY)
    ref = (tX.grad.numpy(), tA.grad.numpy(), tB.grad.numpy())
    return all(np.max(np.abs(np.asarray(g) - r)) < 1e-10 for g, r in zip(got, ref))


def pin_backward_split_invariance(back_fn):
    """The gradients do not depend on how many shards the MLP is split into."""
    M, D, F = 4, 6, 24
    X, A, B, dY = _rand((M, D), 21), _rand((D, F), 22, 0.4), _rand((F, D), 23, 0.4), _rand((M, D), 24)
    ref = back_fn(X, A, B, 1, dY)
    for n in (2, 3, 4, 6, 8, 12, 24):
        got = back_fn(X, A, B, n, dY)
        if not all(np.max(np.abs(np.asarray(g) - r)) < 1e-10 for g, r in zip(got, ref)):
            return False
    return True


# ---------------------------------------------------------------------------
# the oracle passes its pins
# ---------------------------------------------------------------------------

def test_gelu_grad_pins():
    assert pin_gelu_grad_fd(oracle.gelu_grad)
    assert pin_gelu_grad_limits(oracle.gelu_grad)
    assert pin_gelu_grad_torch(oracle.gelu_grad)
    xs = np.linspace(-5, 5, 41)
    assert np.allclose([oracle.gelu_grad_scalar(v) for v in xs], oracle.gelu_grad(xs), rtol=0, atol=1e-13)


@pytest.mark.parametrize("impl", ["numpy", "loops"])
def test_backward_pins(impl):
    fn = oracle.tp_mlp_backward_full if impl == "numpy" else oracle.tp_mlp_backward_loops
    assert pin_backward_fd(fn)
    assert pin_backward_torch(fn)
    if impl == "numpy":
        assert pin_backward_split_invariance(fn)


def test_backward_shard_lists_match_full():
    M, D, F, n = 6, 5, 12, 3
    X, A, B, dY = _rand((M, D), 31), _rand((D, F), 32), _rand((F, D), 33), _rand((M, D), 34)
    dX, dA_l, dB_l = oracle.tp_mlp_backward(X, oracle.shard_mlp(A, B, n), dY)
    dX2, dA, dB = oracle.tp_mlp_backward_full(X, A, B, n, dY)
    assert np.array_equal(dX, dX2)
    w = F // n
    for i in range(n):
        assert np.array_equal(dA_l[i], dA[:, i * w:(i + 1) * w])
        assert np.array_equal(dB_l[i], dB[i * w:(i + 1) * w])


# ---------------------------------------------------------------------------
# planted mistakes are caught
# ---------------------------------------------------------------------------

def _backward_with(grad_fn=oracle.gelu_grad, drop_last_dx=False, da_from_h=False, db_from_s=False,
                   dx_wrong_weight=False):
    def back(X, A, B, n, dY):
        X, A, B, dY = (np.asarray(v, float) for v in (X, A, B, dY))
        dX = np.zeros_like(X)
        dAs, dBs = [], []
        for i, (A_i, B_i) in enumerate(oracle.shard_mlp(A, B, n)):
            S = X @ A_i
            H = oracle.gelu(S)
            dBs.append((S if db_from_s else H).T @ dY)
            dS = (dY @ B_i.T) * grad_fn(S)
            dAs.append(X.T @ (H if da_from_h else dS))
            if not (drop_last_dx and i == n - 1):
                dX = dX + dS @ (B_i if dx_wrong_weight else A_i.T)
        return dX, np.concatenate(dAs, 1), np.concatenate(dBs, 0)
    return back


def test_pins_reject_planted_mistakes():
    assert pin_backward_fd(_backward_with()) and pin_backward_torch(_backward_with())

    def grad_no_second_term(x):
        x = np.asarray(x, float)
        return 0.5 * (1 + np.tanh(oracle.SQRT_2_OVER_PI * (x + oracle.GELU_CUBIC * x ** 3)))

    def grad_no_cubic_factor(x):
        x = np.asarray(x, float)
        t = np.tanh(oracle.SQRT_2_OVER_PI * (x + oracle.GELU_CUBIC * x ** 3))
        return 0.5 * (1 + t) + 0.5 * x * (1 - t * t) * oracle.SQRT_2_OVER_PI

    def grad_erf(x):
        return np.vectorize(lambda v: 0.5 * (1 + math.erf(v / math.sqrt(2))) +
                            v * math.exp(-v * v / 2) / math.sqrt(2 * math.pi))(x)

    for bad in (grad_no_second_term, grad_no_cubic_factor, grad_erf):
        assert not (pin_gelu_grad_fd(bad) and pin_gelu_grad_torch(bad)), bad.__name__
        assert not pin_backward_torch(_backward_with(grad_fn=bad)), bad.__name__

    for kw in ({"drop_last_dx": True}, {"da_from_h": True}, {"db_from_s": True}):
        b = _backward_with(**kw)
        assert not (pin_backward_fd(b) and pin_backward_torch(b) and pin_backward_split_invariance(b)), kw
    # a weight of the wrong shape for dX fails outright or at a pin
    D_eq_w = _backward_with(dx_wrong_weight=True)
    try:
        caught = not pin_backward_torch(D_eq_w)
    except ValueError:
        caught = True
    assert caught
