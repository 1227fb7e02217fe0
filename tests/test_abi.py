"""C-ABI checks that need no GPU.

The library must load, export every function include/tpmlp.h declares, and
reject bad arguments before making any HIP call (so fake but aligned device
addresses are safe here: validation fails first).
"""

import ctypes
import os
import re

import pytest

import tensor_transformer_mlp_tpmlp_amd as tp
from tensor_transformer_mlp_tpmlp_amd import tpmlp as binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpmlp.h")

OK, NULL, SHAPE, INDIV, DTYPE, WS, ALIGN, HIP = range(8)
FAKE = 0x10000  # aligned non-NULL address, never dereferenced by these tests
FAKE2 = 0x20000


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(tpmlp_[a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    return tp.lib()


def test_header_declares_the_page_api():
    names = _declared_functions()
    for required in ("tpmlp_gelu", "tpmlp_shard", "tpmlp_forward"):
        assert required in names
    assert len(names) >= 14


def test_every_declared_symbol_is_exported(L):
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_binding_covers_every_declared_symbol():
    assert sorted(binding.SIGNATURES) == _declared_functions()


def test_status_strings(L):
    for code in range(8):
        s = L.tpmlp_status_string(code).decode()
        assert s.startswith("TPMLP_") and binding.STATUS_NAMES[code] in s
    assert "UNKNOWN" in L.tpmlp_status_string(99).decode()
    assert b"gfx950" in L.tpmlp_version()


def test_gelu_validation(L):
    assert L.tpmlp_gelu(FAKE, FAKE, 0, 1, None) == OK  # empty: no-op, no HIP call
    assert L.tpmlp_gelu(FAKE, FAKE, -1, 1, None) == SHAPE
    assert L.tpmlp_gelu(FAKE, FAKE, 10, 5, None) == DTYPE
    assert L.tpmlp_gelu(None, FAKE, 10, 0, None) == NULL
    assert L.tpmlp_gelu(FAKE, None, 10, 0, None) == NULL
    assert L.tpmlp_gelu(FAKE + 2, FAKE, 10, 1, None) == ALIGN


def test_shard_bytes(L):
    # A^T and B^T, each rounded up to 256 bytes, then F fp32 column sums
    # A^T, B^T, the column sums of A, then A and B as given: 256-byte segments
    assert L.tpmlp_shard_bytes(2, 4, 2, 0) == 5 * 256
    assert L.tpmlp_shard_bytes(4096, 16384, 8, 1) == 4 * 4096 * 16384 * 2 + 16384 * 4
    assert L.tpmlp_shard_bytes(3, 5, 1, 0) == 5 * 256
    for bad in [(0, 4, 2, 0), (2, 0, 1, 0), (2, 4, 3, 0), (2, 4, 0, 0), (2, 4, 8, 0), (2, 4, 2, 9)]:
        assert L.tpmlp_shard_bytes(*bad) == 0


def _shard(L, A=FAKE, B=FAKE, D=2, F=4, n=2, dt=0, packed=FAKE2, nbytes=1 << 20):
    h = ctypes.c_void_p(0xDEAD)
    st = L.tpmlp_shard(A, B, D, F, n, dt, packed, nbytes, ctypes.byref(h), None)
    assert h.value is None  # cleared on error
    return st


def test_shard_validation(L):
    assert _shard(L, n=3) == INDIV                    # F % n != 0
    assert _shard(L, F=12, n=5) == INDIV
    assert _shard(L, n=0) == SHAPE
    assert _shard(L, n=-2) == SHAPE
    assert _shard(L, n=5) == SHAPE                    # n > F
    assert _shard(L, D=0) == SHAPE
    assert _shard(L, F=-4) == SHAPE
    assert _shard(L, D=1 << 23) == SHAPE
    assert _shard(L, D=(1 << 21) + 1) == SHAPE          # one past the largest dimension
    assert _shard(L, D=1 << 21) == WS                   # the largest passes the shape check
    assert _shard(L, F=(1 << 21) + 2, n=2) == SHAPE
    assert _shard(L, F=1 << 21, n=2) == WS
    assert _shard(L, dt=2) == DTYPE
    assert _shard(L, A=None) == NULL
    assert _shard(L, B=None) == NULL
    assert _shard(L, packed=None) == NULL
    assert _shard(L, nbytes=100) == WS
    assert _shard(L, A=FAKE + 4) == ALIGN
    assert _shard(L, packed=FAKE2 + 8) == ALIGN
    assert L.tpmlp_shard(FAKE, FAKE, 2, 4, 2, 0, FAKE2, 1 << 20, None, None) == NULL


def test_descriptor_functions_reject_null(L):
    assert L.tpmlp_shard_count(None) == 0
    assert L.tpmlp_shard_info(None, None, None, None, None) == NULL
    assert L.tpmlp_shard_unpack(None, 0, FAKE, FAKE, None) == NULL
    assert L.tpmlp_forward_workspace_bytes(None, 16, 0, 0) == 0
    assert L.tpmlp_set_workspace(None, FAKE, 100) == NULL
    assert L.tpmlp_forward(FAKE, 4, None, FAKE, None) == NULL
    assert L.tpmlp_forward_ex(FAKE, 4, None, FAKE, None, None) == NULL
    assert L.tpmlp_backward_workspace_bytes(None, 16) == 0
    assert L.tpmlp_backward(FAKE, FAKE, 4, None, None, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == NULL
    L.tpmlp_shards_destroy(None)  # must be a no-op


def test_opts_defaults(L):
    o = binding.Opts()
    o.flags = 7
    L.tpmlp_opts_init(ctypes.byref(o))
    assert o.flags == 0 and o.shard_index == -1 and o.y_dtype == -1
    assert abs(o.ln_eps - 1e-5) < 1e-12 and not o.residual and not o.workspace and not o.events


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        tp.gelu(torch.zeros(8))
    with pytest.raises(ValueError):
        tp.shard_mlp(torch.zeros(2, 4), torch.zeros(4, 2), 2)


def test_attention_pack_validation(L):
    mib = 1 << 20
    assert L.tpmlp_attn_pack_bytes(1024, 16, 4, 1, 0) == 6 * mib + 12288
    assert L.tpmlp_attn_pack_bytes(1024, 16, 4, 1, 1) == 8 * mib + 12288
    assert L.tpmlp_attn_pack_bytes(64, 1, 1, 1, 0) == 3 * 64 * 64 * 2 + 768
    for bad in [(1024, 16, 4, 0, 0), (1000, 16, 4, 1, 0), (1024, 16, 3, 1, 0), (1024, 16, 0, 1, 0),
                (1024, 0, 1, 1, 0), (128, 1, 1, 1, 0)]:
        assert L.tpmlp_attn_pack_bytes(*bad) == 0, bad

    def pack(Wq=FAKE, Wo=None, h=128, heads=2, p=2, dt=1, packed=FAKE2, nbytes=1 << 20):
        out = ctypes.c_void_p(0xDEAD)
        st = L.tpmlp_attn_pack(Wq, FAKE, FAKE, Wo, h, heads, p, dt, packed, nbytes, ctypes.byref(out), None)
        assert out.value is None  # cleared on error
        return st

    assert pack(dt=0) == DTYPE
    assert pack(h=100) == SHAPE
    assert pack(heads=0) == SHAPE
    assert pack(p=3, heads=2) == INDIV
    assert pack(Wq=None) == NULL
    assert pack(packed=None) == NULL
    assert pack(nbytes=1000) == WS
    assert pack(Wq=FAKE + 8) == ALIGN
    assert pack(Wo=FAKE + 4) == ALIGN
    assert L.tpmlp_attn_pack(FAKE, FAKE, FAKE, None, 128, 2, 2, 1, FAKE2, 1 << 20, None, None) == NULL
    assert L.tpmlp_attn_workspace_bytes(None, 2, 8) == 0
    assert L.tpmlp_attention(FAKE, 2, 8, None, FAKE, 0, 0.0, FAKE, 1 << 20, None, None) == NULL
    L.tpmlp_attn_destroy(None)
