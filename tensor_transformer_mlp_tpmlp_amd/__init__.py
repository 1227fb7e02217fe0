"""MI355X-native tensor-parallel MLP: Y = sum_i GeLU_tanh(X A_i) B_i.

Hand-written gfx950 HIP kernels behind the C ABI of include/tpmlp.h; this
package holds the kernels' sources (csrc/), the build script and the thin
ctypes binding.
"""

from .tpmlp import (  # noqa: F401
    ATTN_LAYERNORM,
    ATTN_RESIDUAL,
    AttnWeights,
    BF16,
    F32,
    LIB_PATH,
    OPT_LAYERNORM,
    OPT_LAYERNORM_AFTER,
    Shards,
    TpmlpError,
    attention,
    block,
    gelu,
    lib,
    shard_attention,
    shard_mlp,
    tp_mlp,
    tp_mlp_backward,
)
