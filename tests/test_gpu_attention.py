"""GPU parity of the attention half (tpmlp_attention) against the fp64
oracle ``oracle.attention_oracle.attention_half``, through the C ABI.

The output with the residual is compared together with the attention term
alone (residual off), so that x cannot mask an attention error.  Shapes
cover one token, sequences shorter than a key tile, ragged tiles, several
tiles, 32 and 64 query rows per wave, both output forms (concatenated heads;
row-parallel W^O) and the attention workloads at their full sizes.
"""

import ctypes

import numpy as np
import pytest
import torch

import workloads
import tensor_transformer_mlp_tpmlp_amd as tp
from oracle import attention_oracle as ao
from parity_util import assert_close, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tp.lib()
    yield
    torch.cuda.synchronize()


def _dev_inputs(inp):
    return [to_dev(a, torch.bfloat16) for a in (inp.x, inp.Wq, inp.Wk, inp.Wv, inp.Wo)]


def _check(inp, batch, seq, heads, p, with_wo, layernorm, what):
    x, Wq, Wk, Wv, Wo = _dev_inputs(inp)
    aw = tp.shard_attention(Wq, Wk, Wv, heads, p, Wo=Wo if with_wo else None)
    args = (inp.x, inp.Wq, inp.Wk, inp.Wv, heads, p, batch, seq)
    kw = {"Wo": inp.Wo if with_wo else None, "layernorm": layernorm}
    out = tp.attention(x, batch, seq, aw, layernorm=layernorm, residual=True)
    attn = tp.attention(x, batch, seq, aw, layernorm=layernorm, residual=False)
    torch.cuda.synchronize()
    assert_close(to_f64(out), ao.attention_half(*args, residual=True, **kw), "bf16", f"{what}: x + attn")
    assert_close(to_f64(attn), ao.attention_half(*args, residual=False, **kw), "bf16", f"{what}: attn alone")
    return out, attn, aw, x


# Weights ~ N(0, 1/h): unit-variance projections of the normalised x, so the
# scores q.k / sqrt(d) have standard deviation about 1.
ATTN_SHAPES = [
    # (batch, seq, heads, p, sw scale)
    (1, 1, 1, 1, 1.0),       # one token: softmax of one key
    (2, 5, 2, 2, 1.0),       # shorter than a tile
    (2, 64, 4, 2, 1.0),      # exactly one tile
    (3, 100, 4, 4, 1.0),     # two tiles, ragged, rows not 16-byte aligned in token count
    (2, 136, 2, 1, 1.0),     # three tiles, ragged
    (3, 200, 2, 2, 1.0),     # four tiles, ragged
    (2, 300, 4, 2, 1.0),     # five tiles
    (1, 512, 2, 1, 1.0),     # eight full tiles, one sequence (reads run past the last token)
    (1, 1024, 2, 2, 1.0),    # 64 query rows per wave
    (2, 1100, 1, 1, 1.0),    # 64 query rows per wave, ragged
]


@pytest.mark.parametrize("batch,seq,heads,p,sws", ATTN_SHAPES)
@pytest.mark.parametrize("with_wo", [False, True])
def test_attention_shapes(batch, seq, heads, p, sws, with_wo):
    h = 64 * heads
    say(f"attention b={batch} s={seq} H={heads} p={p} Wo={with_wo}")
    inp = workloads.attn_case(batch, seq, h, seed=40 + seq + heads, sx=1.5, sw=sws / np.sqrt(h))
    inp.x[:] = workloads.round_to_bf16(inp.x + 0.5)  # a non-zero row mean for the LayerNorm
    _check(inp, batch, seq, heads, p, with_wo, True, f"b={batch} s={seq} H={heads}")


@pytest.mark.parametrize("seq", [100, 136])
def test_attention_peaked_scores_exact_projections(seq):
    """Scores with standard deviation about 11, where the softmax is nearly
    one-hot.  With real-valued inputs the bf16 storage of Q, K and V alone
    would move such a softmax by a few percent, so here x is drawn from
    {-1, 0, 1} and the weights from {-1/4, 0, 1/4}, without the LayerNorm:
    every projection is then a multiple of 1/4 below 2^6 in magnitude, exact
    in fp32 and in bf16, and so are the scores.  What remains is the
    kernel's own arithmetic (exp2, P rounded to bf16, fp32 sums), compared
    with the fp64 oracle at the usual bound."""
    batch, heads, p = 3, 4, 4
    h = 64 * heads
    say(f"peaked scores b={batch} s={seq} H={heads}, exact projections")
    rng = np.random.default_rng(77)
    x = rng.integers(-1, 2, size=(batch * seq, h)).astype(np.float32)
    W = [rng.integers(-1, 2, size=(h, h)).astype(np.float32) * 0.25 for _ in range(3)]
    xd, Wq, Wk, Wv = (to_dev(a, torch.bfloat16) for a in (x, *W))
    aw = tp.shard_attention(Wq, Wk, Wv, heads, p)
    attn = tp.attention(xd, batch, seq, aw, layernorm=False, residual=False)
    torch.cuda.synchronize()
    ref = ao.attention_half(x, *W, heads, p, batch, seq, layernorm=False, residual=False)
    S = (x.astype(np.float64) @ W[0])[:seq, :64] @ (x.astype(np.float64) @ W[1])[:seq, :64].T / 8.0
    say(f"score standard deviation {S.std():.1f}, largest {np.abs(S).max():.0f}")
    assert S.std() > 5.0
    assert_close(to_f64(attn), ref, "bf16", "peaked scores, exact projections")


def test_attention_without_layernorm():
    say("attention without LayerNorm")
    inp = workloads.attn_case(2, 96, 256, seed=3, sw=1.0 / 16)
    _check(inp, 2, 96, 4, 2, False, False, "no LayerNorm")


@pytest.mark.parametrize("s", [128, 256, 512])
def test_attention_workloads_full(s):
    w = workloads.ATTN_WORKLOADS[f"attn_s{s}_bf16"]
    say(f"{w.name}: {w.note}")
    inp = workloads.make_attn_inputs(w)
    out, _, aw, x = _check(inp, w.batch, w.seq, w.heads, w.p, False, True, w.name)
    # bit-identical on a second call
    out2 = tp.attention(x, w.batch, w.seq, aw)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_attention_workload_with_out_projection():
    w = workloads.ATTN_WORKLOADS["attn_s256_bf16"]
    say(f"{w.name} with the row-parallel output projection")
    inp = workloads.make_attn_inputs(w)
    _check(inp, w.batch, w.seq, w.heads, w.p, True, True, w.name + " + W^O")


def test_attention_empty_and_errors():
    say("attention: empty input and error paths")
    inp = workloads.attn_case(2, 16, 128, seed=5)
    x, Wq, Wk, Wv, Wo = _dev_inputs(inp)
    aw = tp.shard_attention(Wq, Wk, Wv, 2, 2)
    L = tp.lib()
    nbytes = L.tpmlp_attn_workspace_bytes(aw.handle, 2, 16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    call = lambda xp, b, s, flags, wsb: L.tpmlp_attention(xp, b, s, aw.handle, out.data_ptr(), flags, 0.0,
                                                          ws.data_ptr(), wsb, None, None)
    assert call(x.data_ptr(), 0, 16, 3, nbytes) == 0      # nothing to do
    assert call(x.data_ptr(), 2, 0, 3, nbytes) == 0
    assert call(x.data_ptr(), -1, 16, 3, nbytes) == 2
    assert call(x.data_ptr(), 2, 16, 4, nbytes) == 2      # unknown flag
    assert call(x.data_ptr(), 2, 16, 3, nbytes - 1) == 5
    assert call(x.data_ptr() + 2, 2, 16, 3, nbytes) == 6
    assert call(None, 2, 16, 3, nbytes) == 1
    assert call(x.data_ptr(), 2, 16, 3, nbytes) == 0
    torch.cuda.synchronize()
    ref = ao.attention_half(inp.x, inp.Wq, inp.Wk, inp.Wv, 2, 2, 2, 16)
    assert_close(to_f64(out), ref, "bf16", "through the C ABI")
    with pytest.raises(tp.TpmlpError):
        tp.shard_attention(Wq, Wk, Wv, 3, 1)              # h != 64 * heads
    with pytest.raises(tp.TpmlpError):
        tp.shard_attention(Wq, Wk, Wv, 2, 3)              # p does not divide heads
    with pytest.raises(tp.TpmlpError):
        tp.shard_attention(*(W.float() for W in (Wq, Wk, Wv)), 2, 2)  # fp32 weights


def test_attention_ragged_last_sequence_reads_nothing_past_qkv():
    """The last sequence's last key tile is partial (s = 100: rows 64..127
    of a 100-row sequence).  Rows past the end of Q|K|V must read as zero,
    not as whatever follows it.  Without W^O and on the ragged-M projection
    path (no split scratch) Q|K|V is the last workspace segment; the
    workspace here is one key tile longer than asked for, and that tail
    (like all of it) starts as 0xFF bytes, NaN in bf16.  A value row read
    from there would put NaN into every query row of its head (P = 0 times
    NaN), so the output must be finite and match the oracle."""
    batch, seq, heads, p = 2, 100, 4, 2
    h = 64 * heads
    say(f"attention ragged last sequence b={batch} s={seq} H={heads}, NaN tail after Q|K|V")
    inp = workloads.attn_case(batch, seq, h, seed=808, sw=1.0 / np.sqrt(h))
    x, Wq, Wk, Wv, _ = _dev_inputs(inp)
    aw = tp.shard_attention(Wq, Wk, Wv, heads, p)
    L = tp.lib()
    nbytes = L.tpmlp_attn_workspace_bytes(aw.handle, batch, seq)
    tail = 64 * 3 * h * 2
    ws = torch.full((nbytes + tail,), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream().cuda_stream
    for flags in (0, 3):
        st = L.tpmlp_attention(x.data_ptr(), batch, seq, aw.handle, out.data_ptr(), flags, 0.0, ws.data_ptr(),
                               nbytes, None, stream)
        assert st == 0
        torch.cuda.synchronize()
        # the tail was not written
        assert bool((ws[nbytes:] == 0xFF).all())
        ref = ao.attention_half(inp.x, inp.Wq, inp.Wk, inp.Wv, heads, p, batch, seq,
                                layernorm=bool(flags & 1), residual=bool(flags & 2))
        assert_close(to_f64(out), ref, "bf16", f"ragged last sequence, flags={flags}")
