"""Pins of the attention oracle (CPU only).

The oracle of the attention half is pinned against closed forms (uniform
attention averages V, a single key returns its value), invariants (softmax
rows sum to one and ignore a shift, key/value permutations, the TP size p
only groups heads, sequences are independent) and library routines in
float64 (torch's softmax, scaled_dot_product_attention and layer_norm).  A
set of plausible mistakes, planted in copies of the oracle's functions, must
each fail at least one pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention_oracle as ao

F = torch.nn.functional


def _rng(seed):
    return np.random.default_rng(seed)


def _weights(h, seed, scale=None):
    r = _rng(seed)
    s = 1.0 / math.sqrt(h) if scale is None else scale
    return [r.standard_normal((h, h)) * s for _ in range(4)]


def _torch_half(x, Wq, Wk, Wv, H, batch, seq, Wo=None, layernorm=True, residual=True):
    """The attention half with torch ops in float64 (heads moved before the
    token axis, then torch's scaled_dot_product_attention)."""
    xt = torch.from_numpy(x)
    h = x.shape[1]
    d = h // H
    xn = F.layer_norm(xt, (h,)) if layernorm else xt

    def heads(W):
        return (xn @ torch.from_numpy(W)).view(batch, seq, H, d).transpose(1, 2)

    o = F.scaled_dot_product_attention(heads(Wq), heads(Wk), heads(Wv))
    cat = o.transpose(1, 2).reshape(batch * seq, h)
    attn = cat if Wo is None else cat @ torch.from_numpy(Wo)
    return (xt + attn if residual else attn).numpy()


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_softmax(sm):
    z = _rng(1).standard_normal((5, 9)) * 4.0
    ok = float(np.max(np.abs(sm(z) - torch.softmax(torch.from_numpy(z), -1).numpy()))) <= 1e-15
    ok &= bool(np.all(np.abs(sm(z).sum(axis=-1) - 1.0) <= 1e-14))
    ok &= float(np.max(np.abs(sm(z + 123.0) - sm(z)))) <= 1e-13
    big = sm(np.array([[1000.0, 999.0, 0.0]]))
    ok &= bool(np.all(np.isfinite(big))) and abs(big[0, 0] - 1.0 / (1.0 + math.exp(-1.0))) <= 1e-15
    return bool(ok)


def pin_head_attention(att):
    r = _rng(2)
    K, V = r.standard_normal((7, 8)), r.standard_normal((7, 5))
    # zero queries attend uniformly: the mean of the values
    ok = float(np.max(np.abs(att(np.zeros((3, 8)), K, V) - V.mean(axis=0)))) <= 1e-15
    # a single key returns its value whatever the query
    ok &= float(np.max(np.abs(att(r.standard_normal((4, 8)), K[:1], V[:1]) - V[:1]))) <= 1e-15
    # torch's scaled_dot_product_attention (scale 1/sqrt(d)) in float64
    Q = r.standard_normal((6, 8)) * 2.0
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(a)[None] for a in (Q, K, V)))[0].numpy()
    ok &= float(np.max(np.abs(att(Q, K, V) - ref))) <= 1e-14
    # permuting keys and values together changes nothing
    perm = r.permutation(7)
    ok &= float(np.max(np.abs(att(Q, K[perm], V[perm]) - att(Q, K, V)))) <= 1e-14
    # a query aligned with one of several orthogonal keys, scaled up, selects its value
    Ko = np.eye(8)[:4] * 10.0
    Vo = r.standard_normal((4, 3))
    ok &= float(np.max(np.abs(att(Ko[2:3] * 10.0, Ko, Vo) - Vo[2]))) <= 1e-12
    return bool(ok)


def pin_attention_half(half, batch=2, seq=5, h=16, H=4):
    x = _rng(3).standard_normal((batch * seq, h)) * 1.5 + 0.5
    Wq, Wk, Wv, Wo = _weights(h, 4, scale=0.6)
    ok = True
    for kw in ({}, {"Wo": Wo}, {"layernorm": False}, {"residual": False}, {"Wo": Wo, "residual": False}):
        ref = _torch_half(x, Wq, Wk, Wv, H, batch, seq, **kw)
        for p in (1, 2, 4):
            got = half(x, Wq, Wk, Wv, H, p, batch, seq, **kw)
            ok &= float(np.max(np.abs(got - ref))) <= 1e-12 * max(1.0, float(np.max(np.abs(ref))))
    # an identity output projection is the concatenation
    ok &= float(np.max(np.abs(half(x, Wq, Wk, Wv, H, 2, batch, seq, Wo=np.eye(h))
                              - half(x, Wq, Wk, Wv, H, 2, batch, seq)))) <= 1e-13
    # sequences are independent: changing the second does not move the first
    x2 = x.copy()
    x2[seq:] += 3.0
    a, b = half(x, Wq, Wk, Wv, H, 2, batch, seq), half(x2, Wq, Wk, Wv, H, 2, batch, seq)
    ok &= bool(np.array_equal(a[:seq], b[:seq]))
    return bool(ok)


# ---------------------------------------------------------------------------
# the oracle passes every pin
# ---------------------------------------------------------------------------

def test_softmax():
    assert pin_softmax(ao.softmax)
    row = [0.5, -1.0, 2.0]
    assert max(abs(a - b) for a, b in zip(ao.softmax_loops(row), ao.softmax(np.array(row)))) <= 1e-16


def test_head_attention():
    assert pin_head_attention(ao.head_attention)


def test_attention_half():
    assert pin_attention_half(ao.attention_half)


def test_loops_agree_with_numpy():
    batch, seq, h, H = 2, 3, 8, 2
    x = _rng(5).standard_normal((batch * seq, h))
    Wq, Wk, Wv, Wo = _weights(h, 6)
    for kw in ({}, {"Wo": Wo}, {"layernorm": False, "residual": False}):
        a = np.array(ao.attention_half_loops(x.tolist(), Wq.tolist(), Wk.tolist(), Wv.tolist(), H, 2, batch, seq,
                                             **{k: (v.tolist() if isinstance(v, np.ndarray) else v)
                                                for k, v in kw.items()}))
        b = ao.attention_half(x, Wq, Wk, Wv, H, 2, batch, seq, **kw)
        assert np.max(np.abs(a - b)) <= 1e-13


def test_divisibility_rules():
    x = np.zeros((4, 12))
    W = np.zeros((12, 12))
    with pytest.raises(ValueError):
        ao.attention_half(x, W, W, W, 5, 1, 1, 4)     # h not divisible by H
    with pytest.raises(ValueError):
        ao.attention_half(x, W, W, W, 4, 3, 1, 4)     # H not divisible by p
    with pytest.raises(ValueError):
        ao.attention_half(x, W, W, W, 4, 2, 2, 4)     # rows != batch*seq


# ---------------------------------------------------------------------------
# planted mistakes must be caught
# ---------------------------------------------------------------------------

def _half_with(head_fn=None, over_heads=False, whole_batch=False, residual_of_normed=False,
               wo_columns=False, no_residual=False, no_layernorm=False):
    """A copy of the attention half with one planted mistake."""
    head_fn = head_fn or ao.head_attention

    def half(x, Wq, Wk, Wv, H, p, batch, seq, Wo=None, layernorm=True, residual=True):
        x = np.asarray(x, float)
        h = x.shape[1]
        d = h // H
        xn = oracle.layer_norm(x) if (layernorm and not no_layernorm) else x
        Q, K, V = xn @ Wq, xn @ Wk, xn @ Wv
        cat = np.zeros_like(x)
        if over_heads:
            # the printed code taken literally: attention across the heads of each token
            for t in range(x.shape[0]):
                q, k, v = (A[t].reshape(H, d) for A in (Q, K, V))
                cat[t] = head_fn(q, k, v).reshape(h)
        else:
            groups = [slice(0, batch * seq)] if whole_batch else [slice(b * seq, (b + 1) * seq)
                                                                 for b in range(batch)]
            for j in range(H):
                c = slice(j * d, (j + 1) * d)
                for rows in groups:
                    cat[rows, c] = head_fn(Q[rows, c], K[rows, c], V[rows, c])
        attn = cat
        if Wo is not None:
            attn = cat @ (Wo.T if wo_columns else Wo)
        base = xn if residual_of_normed else x
        return base + attn if (residual and not no_residual) else attn

    return half


def test_pins_reject_planted_mistakes():
    # the hand-made copy passes when unbroken
    assert pin_attention_half(_half_with())

    def no_scale(Q, K, V):
        return ao.softmax(np.asarray(Q) @ np.asarray(K).T) @ np.asarray(V)

    def scale_by_d(Q, K, V):
        return ao.softmax((np.asarray(Q) @ np.asarray(K).T) / Q.shape[-1]) @ np.asarray(V)

    def softmax_over_queries(Q, K, V):
        return ao.softmax((np.asarray(Q) @ np.asarray(K).T) / math.sqrt(Q.shape[-1]), axis=0) @ np.asarray(V)

    def keys_as_queries(Q, K, V):
        return ao.softmax((np.asarray(Q) @ np.asarray(Q).T) / math.sqrt(Q.shape[-1])) @ np.asarray(V)

    for bad in (no_scale, scale_by_d, softmax_over_queries):
        assert not pin_head_attention(bad), bad.__name__
        assert not pin_attention_half(_half_with(head_fn=bad)), bad.__name__
    assert not pin_attention_half(_half_with(head_fn=keys_as_queries))

    def softmax_no_shift_wrong_axis(z, axis=-1):
        with np.errstate(over="ignore", invalid="ignore"):
            e = np.exp(np.asarray(z, float))
            return e / e.sum(axis=0, keepdims=True)

    assert not pin_softmax(softmax_no_shift_wrong_axis)

    for name, kw in {"attention over heads": {"over_heads": True},
                     "sequences not separated": {"whole_batch": True},
                     "residual of the normalised x": {"residual_of_normed": True},
                     "W^O by columns": {"wo_columns": True},
                     "no residual": {"no_residual": True},
                     "no LayerNorm": {"no_layernorm": True}}.items():
        assert not pin_attention_half(_half_with(**kw)), name
