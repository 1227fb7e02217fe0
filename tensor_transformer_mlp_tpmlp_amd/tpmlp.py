"""Python binding of libtpmlp.so (argument marshalling only).

The names follow "Tensor-Parallel MLP (Megatron)", section "What to
implement": ``gelu(x)``, ``shard_mlp(A, B, n)`` and ``tp_mlp(X, shards)``.
Every step of the computation runs in the HIP kernels behind the C ABI
(include/tpmlp.h); this module only allocates outputs and workspaces with
torch on the tensors' device and passes raw device pointers and the current
stream.  There is no fallback: if the library is not built, or a tensor is
not on a GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence, Tuple

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libtpmlp.so")

F32, BF16 = 0, 1
OPT_LAYERNORM = 1
OPT_LAYERNORM_AFTER = 2
ATTN_LAYERNORM = 1
ATTN_RESIDUAL = 2
STATUS_NAMES = {
    0: "TPMLP_OK", 1: "TPMLP_ERR_NULL", 2: "TPMLP_ERR_SHAPE", 3: "TPMLP_ERR_INDIVISIBLE",
    4: "TPMLP_ERR_DTYPE", 5: "TPMLP_ERR_WORKSPACE", 6: "TPMLP_ERR_ALIGN", 7: "TPMLP_ERR_HIP",
}

# every function declared in include/tpmlp.h, with its ctypes signature
_c_i64, _c_int, _c_vp, _c_sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t


class Opts(ctypes.Structure):
    """Mirror of tpmlp_opts."""
    _fields_ = [("flags", ctypes.c_int), ("ln_eps", ctypes.c_float), ("y_dtype", ctypes.c_int),
                ("residual", ctypes.c_void_p), ("shard_index", ctypes.c_int),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("events", ctypes.c_void_p), ("save_preact", ctypes.c_void_p),
                ("save_act", ctypes.c_void_p)]


SIGNATURES = {
    "tpmlp_status_string": (ctypes.c_char_p, [_c_int]),
    "tpmlp_version": (ctypes.c_char_p, []),
    "tpmlp_gelu": (_c_int, [_c_vp, _c_vp, _c_i64, _c_int, _c_vp]),
    "tpmlp_shard_bytes": (_c_sz, [_c_i64, _c_i64, _c_int, _c_int]),
    "tpmlp_shard": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_int, _c_vp, _c_sz,
                             ctypes.POINTER(_c_vp), _c_vp]),
    "tpmlp_shard_count": (_c_int, [_c_vp]),
    "tpmlp_shard_info": (_c_int, [_c_vp, ctypes.POINTER(_c_i64), ctypes.POINTER(_c_i64),
                                  ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
    "tpmlp_shard_unpack": (_c_int, [_c_vp, _c_int, _c_vp, _c_vp, _c_vp]),
    "tpmlp_shards_destroy": (None, [_c_vp]),
    "tpmlp_forward_workspace_bytes": (_c_sz, [_c_vp, _c_i64, _c_int, _c_int]),
    "tpmlp_set_workspace": (_c_int, [_c_vp, _c_vp, _c_sz]),
    "tpmlp_forward": (_c_int, [_c_vp, _c_i64, _c_vp, _c_vp, _c_vp]),
    "tpmlp_opts_init": (None, [ctypes.POINTER(Opts)]),
    "tpmlp_forward_ex": (_c_int, [_c_vp, _c_i64, _c_vp, _c_vp, ctypes.POINTER(Opts), _c_vp]),
    "tpmlp_forward_noalloc": (_c_int, [_c_vp, _c_i64, _c_vp, _c_vp, ctypes.POINTER(Opts), _c_vp]),
    "tpmlp_backward_workspace_bytes": (_c_sz, [_c_vp, _c_i64]),
    "tpmlp_backward": (_c_int, [_c_vp, _c_vp, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz,
                                _c_vp]),
    "tpmlp_attn_pack_bytes": (_c_sz, [_c_i64, _c_int, _c_int, _c_int, _c_int]),
    "tpmlp_attn_pack": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_int, _c_int, _c_int, _c_vp, _c_sz,
                                 ctypes.POINTER(_c_vp), _c_vp]),
    "tpmlp_attn_destroy": (None, [_c_vp]),
    "tpmlp_attn_workspace_bytes": (_c_sz, [_c_vp, _c_i64, _c_i64]),
    "tpmlp_attention": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_int, ctypes.c_float, _c_vp, _c_sz,
                                 _c_vp, _c_vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m tensor_transformer_mlp_tpmlp_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class TpmlpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().tpmlp_status_string(status).decode()
        super().__init__(f"{where}: {msg}")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise TpmlpError(status, where)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.float32 if code == F32 else torch.bfloat16


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class _StreamWorkspaces:
    """Grow-only device workspaces, one per stream.  Calls on one stream run
    in order and can share a workspace; calls on different streams may
    overlap, so each stream gets its own."""

    def __init__(self, device: torch.device):
        self.device = device
        self._by_stream: Dict[int, torch.Tensor] = {}

    def get(self, nbytes: int, stream: int) -> torch.Tensor:
        ws = self._by_stream.get(stream)
        if ws is None or ws.numel() < nbytes:
            # allocated on the current stream, which is `stream`
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self._by_stream[stream] = ws
        return ws


def gelu(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Elementwise tanh-GeLU on the GPU (tpmlp_gelu)."""
    if out is None:
        out = torch.empty_like(x)
    if out.dtype != x.dtype or out.numel() != x.numel():
        raise ValueError("out must match x in dtype and size")
    _check(lib().tpmlp_gelu(_dev(x, "x"), _dev(out, "out"), x.numel(), _dtype_code(x.dtype),
                            _stream(x.device)), "tpmlp_gelu")
    return out


class Shards:
    """n (A_i, B_i) pairs packed on the GPU (a tpmlp_shards descriptor).

    Holds the packed weight buffer (owned here, as a torch tensor) and a
    grow-only workspace per stream.
    """

    def __init__(self, handle: int, packed: torch.Tensor, D: int, F: int, n: int, dtype: torch.dtype):
        self._handle = handle
        self.packed = packed
        self.D, self.F, self.n, self.dtype = D, F, n, dtype
        self.device = packed.device
        self._ws = _StreamWorkspaces(self.device)

    @property
    def handle(self) -> int:
        return self._handle

    def __len__(self) -> int:
        return self.n

    def pairs(self) -> List[Tuple[torch.Tensor, torch.Tensor]]:
        """Unpack every pair to the page's layout: A_i (D x F/n), B_i (F/n x D)."""
        w = self.F // self.n
        out = []
        for i in range(self.n):
            A_i = torch.empty((self.D, w), dtype=self.dtype, device=self.device)
            B_i = torch.empty((w, self.D), dtype=self.dtype, device=self.device)
            _check(lib().tpmlp_shard_unpack(self._handle, i, A_i.data_ptr(), B_i.data_ptr(),
                                            _stream(self.device)), "tpmlp_shard_unpack")
            out.append((A_i, B_i))
        return out

    def workspace(self, nbytes: int, stream: int) -> torch.Tensor:
        return self._ws.get(nbytes, stream)

    def close(self) -> None:
        if self._handle:
            lib().tpmlp_shards_destroy(self._handle)
            self._handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def shard_mlp(A: torch.Tensor, B: torch.Tensor, n: int) -> Shards:
    """Split A (D x F) by columns and B (F x D) by rows into n pairs (tpmlp_shard)."""
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be matrices")
    D, F = A.shape
    if B.dtype != A.dtype:
        raise TypeError("A and B must have the same dtype")
    if B.shape != (F, D):
        raise ValueError(f"B must be ({F}, {D}), got {tuple(B.shape)}")
    dt = _dtype_code(A.dtype)
    L = lib()
    nbytes = L.tpmlp_shard_bytes(D, F, n, dt)
    packed = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=A.device)
    h = ctypes.c_void_p()
    _check(L.tpmlp_shard(_dev(A, "A"), _dev(B, "B"), D, F, n, dt, packed.data_ptr(), packed.numel(),
                         ctypes.byref(h), _stream(A.device)), "tpmlp_shard")
    return Shards(h.value, packed, D, F, n, A.dtype)


def tp_mlp(X: torch.Tensor, shards: Shards, *, layernorm: bool = False, layernorm_after: bool = False,
           eps: float = 1e-5,
           residual: Optional[torch.Tensor] = None, shard_index: int = -1,
           out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
           events: Optional[Sequence[int]] = None,
           save_preact: Optional[torch.Tensor] = None,
           save_act: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = sum_i GeLU(X A_i) B_i on the GPU (tpmlp_forward_ex).

    layernorm: normalise each row of X first (no affine); layernorm_after:
    normalise each row of residual + Y last instead; residual: added once
    after the shard sum; shard_index: return only partial Y_i; events: four
    hipEvent_t handles recorded around the kernels (timing hook);
    save_preact: an (M, F) tensor (F/n with shard_index) of the weights'
    dtype that receives the pre-activation X A for tp_mlp_backward;
    save_act: the same for the activation H = GeLU(X A) (GEMM1 writes it
    there instead of into the workspace).
    """
    if X.dim() != 2 or X.shape[1] != shards.D:
        raise ValueError(f"X must be (M, {shards.D})")
    if X.dtype != shards.dtype:
        raise TypeError("X must have the weights' dtype")
    M = X.shape[0]
    y_dtype = shards.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((M, shards.D), dtype=y_dtype, device=X.device)
    elif out.dtype != y_dtype or tuple(out.shape) != (M, shards.D):
        raise ValueError("out has the wrong dtype or shape")
    flags = (OPT_LAYERNORM if layernorm else 0) | (OPT_LAYERNORM_AFTER if layernorm_after else 0)
    L = lib()
    nbytes = L.tpmlp_forward_workspace_bytes(shards.handle, M, flags, 1 if shard_index >= 0 else 0)
    stream = _stream(X.device)
    ws = shards.workspace(nbytes, stream)
    o = Opts()
    L.tpmlp_opts_init(ctypes.byref(o))
    o.flags = flags
    o.ln_eps = eps
    o.y_dtype = _dtype_code(y_dtype)
    if residual is not None:
        if residual.dtype != X.dtype or tuple(residual.shape) != (M, shards.D):
            raise ValueError("residual must match X")
        o.residual = _dev(residual, "residual")
    o.shard_index = shard_index
    if save_preact is not None:
        nh = shards.F // shards.n if shard_index >= 0 else shards.F
        if save_preact.dtype != shards.dtype or tuple(save_preact.shape) != (M, nh):
            raise ValueError(f"save_preact must be ({M}, {nh}) with the weights' dtype")
        o.save_preact = _dev(save_preact, "save_preact")
    if save_act is not None:
        nh = shards.F // shards.n if shard_index >= 0 else shards.F
        if save_act.dtype != shards.dtype or tuple(save_act.shape) != (M, nh):
            raise ValueError(f"save_act must be ({M}, {nh}) with the weights' dtype")
        o.save_act = _dev(save_act, "save_act")
    o.workspace = ws.data_ptr()
    o.workspace_bytes = ws.numel()
    ev_arr = None
    if events is not None:
        ev_arr = (ctypes.c_void_p * 4)(*[e or None for e in events])
        o.events = ctypes.cast(ev_arr, ctypes.c_void_p)
    _check(L.tpmlp_forward_ex(_dev(X, "X") if M else X.data_ptr(), M, shards.handle,
                              _dev(out, "out") if M else out.data_ptr(), ctypes.byref(o), stream),
           "tpmlp_forward_ex")
    return out


def tp_mlp_backward(X: torch.Tensor, dY: torch.Tensor, shards: Shards, out=None,
                    preact: Optional[torch.Tensor] = None, act: Optional[torch.Tensor] = None):
    """Gradients (dX, dA, dB) of the TP-MLP given dY = dL/dY (tpmlp_backward).

    dA has A's layout (D x F, shard i in its columns), dB has B's (F x D,
    shard i in its rows); all three in the weights' dtype.  `out` may give
    the three result tensors; `preact` the (M, F) pre-activation a forward
    kept with save_preact (otherwise it is recomputed); `act` the (M, F)
    activation it kept with save_act (otherwise recomputed from preact).
    """
    if X.dim() != 2 or X.shape[1] != shards.D:
        raise ValueError(f"X must be (M, {shards.D})")
    if X.dtype != shards.dtype or dY.dtype != shards.dtype:
        raise TypeError("X and dY must have the weights' dtype")
    if tuple(dY.shape) != tuple(X.shape):
        raise ValueError("dY must have X's shape")
    M = X.shape[0]
    if out is None:
        dX = torch.empty_like(X)
        dA = torch.empty((shards.D, shards.F), dtype=shards.dtype, device=X.device)
        dB = torch.empty((shards.F, shards.D), dtype=shards.dtype, device=X.device)
    else:
        dX, dA, dB = out
        want = ((M, shards.D), (shards.D, shards.F), (shards.F, shards.D))
        if any(tuple(t.shape) != sh or t.dtype != shards.dtype for t, sh in zip((dX, dA, dB), want)):
            raise ValueError("out tensors have the wrong shape or dtype")
    pp = None
    if preact is not None:
        if preact.dtype != shards.dtype or tuple(preact.shape) != (M, shards.F):
            raise ValueError(f"preact must be ({M}, {shards.F}) with the weights' dtype")
        pp = _dev(preact, "preact") if M else None
    ap = None
    if act is not None:
        if act.dtype != shards.dtype or tuple(act.shape) != (M, shards.F):
            raise ValueError(f"act must be ({M}, {shards.F}) with the weights' dtype")
        ap = _dev(act, "act") if M else None
    L = lib()
    nbytes = L.tpmlp_backward_workspace_bytes(shards.handle, M)
    stream = _stream(X.device)
    ws = shards.workspace(nbytes, stream)
    _check(L.tpmlp_backward(_dev(X, "X") if M else X.data_ptr(), _dev(dY, "dY") if M else dY.data_ptr(), M,
                            shards.handle, pp, ap, _dev(dX, "dX") if M else dX.data_ptr(), _dev(dA, "dA"),
                            _dev(dB, "dB"), ws.data_ptr(), ws.numel(), stream), "tpmlp_backward")
    return dX, dA, dB


class AttnWeights:
    """Packed projection weights of the attention half (a tpmlp_attn descriptor).

    Holds the packed buffer (owned here, as a torch tensor) and a grow-only
    workspace per stream.
    """

    def __init__(self, handle: int, packed: torch.Tensor, hidden: int, heads: int, p: int, has_wo: bool):
        self._handle = handle
        self.packed = packed
        self.hidden, self.heads, self.p, self.has_wo = hidden, heads, p, has_wo
        self.device = packed.device
        self._ws = _StreamWorkspaces(self.device)

    @property
    def handle(self) -> int:
        return self._handle

    def workspace(self, nbytes: int, stream: int) -> torch.Tensor:
        return self._ws.get(nbytes, stream)

    def close(self) -> None:
        if self._handle:
            lib().tpmlp_attn_destroy(self._handle)
            self._handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def shard_attention(Wq: torch.Tensor, Wk: torch.Tensor, Wv: torch.Tensor, heads: int, p: int,
                    Wo: Optional[torch.Tensor] = None) -> AttnWeights:
    """Pack W^Q, W^K, W^V (h x h, x W) and optionally W^O for `heads` heads
    over p ranks (tpmlp_attn_pack).  Without W^O the heads' outputs are
    concatenated (all_gather + cat); with it, projected row-parallel."""
    h = Wq.shape[0]
    for name, W in (("Wq", Wq), ("Wk", Wk), ("Wv", Wv)) + ((("Wo", Wo),) if Wo is not None else ()):
        if W.dim() != 2 or tuple(W.shape) != (h, h):
            raise ValueError(f"{name} must be ({h}, {h})")
        if W.dtype != Wq.dtype:
            raise TypeError("the projection weights must share one dtype")
    dt = _dtype_code(Wq.dtype)
    L = lib()
    nbytes = L.tpmlp_attn_pack_bytes(h, heads, p, dt, 1 if Wo is not None else 0)
    packed = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=Wq.device)
    hd = ctypes.c_void_p()
    _check(L.tpmlp_attn_pack(_dev(Wq, "Wq"), _dev(Wk, "Wk"), _dev(Wv, "Wv"),
                             _dev(Wo, "Wo") if Wo is not None else None, h, heads, p, dt, packed.data_ptr(),
                             packed.numel(), ctypes.byref(hd), _stream(Wq.device)), "tpmlp_attn_pack")
    return AttnWeights(hd.value, packed, h, heads, p, Wo is not None)


def attention(x: torch.Tensor, batch: int, seq: int, weights: AttnWeights, *, layernorm: bool = True,
              residual: bool = True, eps: float = 1e-5, out: Optional[torch.Tensor] = None,
              events: Optional[Sequence[int]] = None) -> torch.Tensor:
    """The attention half on the GPU (tpmlp_attention): x is (batch*seq, h),
    sequence b in rows b*seq .. (b+1)*seq-1; events: four hipEvent_t handles
    recorded around the kernels (timing hook)."""
    if x.dim() != 2 or x.shape[1] != weights.hidden or x.shape[0] != batch * seq:
        raise ValueError(f"x must be ({batch * seq}, {weights.hidden})")
    if out is None:
        out = torch.empty_like(x)
    elif out.dtype != x.dtype or out.shape != x.shape:
        raise ValueError("out must match x")
    L = lib()
    stream = _stream(x.device)
    ws = weights.workspace(L.tpmlp_attn_workspace_bytes(weights.handle, batch, seq), stream)
    flags = (ATTN_LAYERNORM if layernorm else 0) | (ATTN_RESIDUAL if residual else 0)
    M = batch * seq
    ev_arr = None
    if events is not None:
        ev_arr = (ctypes.c_void_p * 4)(*[e or None for e in events])
    _check(L.tpmlp_attention(_dev(x, "x") if M else x.data_ptr(), batch, seq, weights.handle,
                             _dev(out, "out") if M else out.data_ptr(), flags, eps, ws.data_ptr(), ws.numel(),
                             ctypes.cast(ev_arr, ctypes.c_void_p) if ev_arr is not None else None, stream),
           "tpmlp_attention")
    return out


def block(x: torch.Tensor, batch: int, seq: int, weights: AttnWeights, shards: Shards, *, eps: float = 1e-5,
          x1: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
          events: Optional[Sequence[int]] = None) -> torch.Tensor:
    """The whole block forward in the code order of "LLM Lab Notes 06",
    section 2, markers 2 to 7: x1 = x + attn(LayerNorm(x)) (tpmlp_attention),
    then out = x1 + TP-MLP(LayerNorm(x1)) (tpmlp_forward_ex).  Two library
    calls on the current stream; x1 (optional) receives the attention half's
    output.  events: three hipEvent_t handles recorded before the attention
    half, between the halves and after the FFN half (segment timing)."""
    if shards.D != weights.hidden or shards.dtype != x.dtype:
        raise ValueError("the FFN weights must have the attention's hidden size and x's dtype")
    if x1 is None:
        x1 = torch.empty_like(x)
    ev = list(events) if events is not None else [None, None, None]
    if len(ev) != 3:
        raise ValueError("events must hold three handles")
    attention(x, batch, seq, weights, layernorm=True, residual=True, eps=eps, out=x1,
              events=[ev[0], None, None, ev[1]])
    return tp_mlp(x1, shards, layernorm=True, eps=eps, residual=x1, out=out, events=[None, None, None, ev[2]])
