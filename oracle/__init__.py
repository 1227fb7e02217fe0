"""fp64 CPU oracle (test infrastructure only; never on the product path)."""

from . import attention_oracle  # noqa: F401

from .tpmlp_oracle import (  # noqa: F401
    GELU_CUBIC,
    LN_EPS,
    SQRT_2_OVER_PI,
    gelu,
    gelu_grad,
    gelu_grad_scalar,
    gelu_scalar,
    layer_norm,
    layer_norm_loops,
    norm_after_ffn,
    norm_after_ffn_loops,
    post_ln_ffn,
    shard_mlp,
    shard_outputs,
    tp_mlp,
    tp_mlp_backward,
    tp_mlp_backward_full,
    tp_mlp_backward_loops,
    tp_mlp_loops,
)
