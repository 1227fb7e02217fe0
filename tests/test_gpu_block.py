"""GPU parity of the whole block forward against the fp64 oracle.

"LLM Lab Notes 06", section 2, markers 2 to 7, in the code's order:
x1 = x + attn(LayerNorm(x)), then out = x1 + TP-MLP(LayerNorm(x1)).  The
GPU side is the binding's ``block`` (tpmlp_attention, then
tpmlp_forward_ex); the reference is the oracle's attention half followed by
its FFN half, both in fp64 with no rounding between them.  The FFN term is
also checked alone, so that the residual x1 cannot mask an FFN error, and
the other placement of the Norm (LayerNorm(x1 + TP-MLP(x1)), the FFN half
with the Norm after the residual) is checked on the same attention output.
"""

import numpy as np
import pytest
import torch

import oracle
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


@pytest.mark.parametrize("s", [128, 256, 512])
def test_block_forward(s):
    wa = workloads.ATTN_WORKLOADS[f"attn_s{s}_bf16"]
    wf = workloads.WORKLOADS[f"postln_s{s}_bf16"]
    say(f"block b={wa.batch} s={s} h={wa.hidden}: attention half then FFN half (F={wf.F}, n={wf.n})")
    ai = workloads.make_attn_inputs(wa)
    fi = workloads.make_inputs(wf)
    bf = torch.bfloat16
    x = to_dev(ai.x, bf)
    aw = tp.shard_attention(to_dev(ai.Wq, bf), to_dev(ai.Wk, bf), to_dev(ai.Wv, bf), wa.heads, wa.p)
    sh = tp.shard_mlp(to_dev(fi.A, bf), to_dev(fi.B, bf), wf.n)
    x1 = torch.empty_like(x)
    out = tp.block(x, wa.batch, wa.seq, aw, sh, x1=x1)
    torch.cuda.synchronize()

    shards = oracle.shard_mlp(fi.A, fi.B, wf.n)
    x1_ref = ao.attention_half(ai.x, ai.Wq, ai.Wk, ai.Wv, wa.heads, wa.p, wa.batch, wa.seq)
    out_ref = oracle.post_ln_ffn(x1_ref, shards)
    assert_close(to_f64(x1), x1_ref, "bf16", f"block s={s}: x1 = x + attn")
    assert_close(to_f64(out), out_ref, "bf16", f"block s={s}: out = x1 + FFN(LN(x1))")
    # the FFN term alone (the residual must not hide it)
    ffn = tp.tp_mlp(x1, sh, layernorm=True)
    torch.cuda.synchronize()
    assert_close(to_f64(ffn), oracle.tp_mlp(oracle.layer_norm(x1_ref), shards), "bf16",
                 f"block s={s}: FFN(LN(x1)) alone")
    # the Norm after the residual, on the same attention output
    out_after = tp.tp_mlp(x1, sh, layernorm_after=True, residual=x1)
    torch.cuda.synchronize()
    assert_close(to_f64(out_after), oracle.norm_after_ffn(x1_ref, shards), "bf16",
                 f"block s={s}: LayerNorm(x1 + FFN(x1))")
    # bit-identical on a second call
    out2 = tp.block(x, wa.batch, wa.seq, aw, sh)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_block_rejects_mismatched_weights():
    say("block: mismatched hidden sizes")
    ai = workloads.attn_case(1, 16, 128, seed=6)
    bf = torch.bfloat16
    aw = tp.shard_attention(to_dev(ai.Wq, bf), to_dev(ai.Wk, bf), to_dev(ai.Wv, bf), 2, 2)
    fi = workloads.random_case(16, 256, 512, seed=6, dtype="bf16")
    sh = tp.shard_mlp(to_dev(fi.A, bf), to_dev(fi.B, bf), 2)
    with pytest.raises(ValueError):
        tp.block(to_dev(ai.x, bf), 1, 16, aw, sh)
