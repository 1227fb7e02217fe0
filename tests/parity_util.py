"""Helpers shared by the GPU parity tests (comparison rules and marshalling)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads

# Tolerances.  fp32 workloads: normwise max-relative error
# max|Y - Y_ref| / max|Y_ref| <= 1e-4.  bf16 workloads with fp32 accumulation:
# max|Y - Y_ref| <= 1e-2 * max|Y_ref|.
TOL_F32 = 1e-4
TOL_BF16 = 1e-2


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(name: str) -> torch.dtype:
    return torch.float32 if name == "f32" else torch.bfloat16


def to_dev(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """float32 array holding storage-type values -> device tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(dtype).contiguous()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def normwise_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (scale if scale > 0 else 1.0)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> float:
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    err = normwise_err(got, ref)
    say(f"{what}: normwise max error {err:.3e} (tolerance {tol:g})")
    assert err <= tol, f"{what}: {err:.3e} > {tol:g}"
    return err


def oracle_forward(X: np.ndarray, A: np.ndarray, B: np.ndarray, n: int, layernorm: bool = False,
                   residual: bool = False, eps: float = oracle.LN_EPS,
                   layernorm_after: bool = False) -> np.ndarray:
    """fp64 oracle of what tp_mlp computes with the given options."""
    shards = oracle.shard_mlp(A, B, n)
    x = X.astype(np.float64)
    if layernorm_after:
        if residual:
            return oracle.norm_after_ffn(x, shards, eps)
        return oracle.layer_norm(oracle.tp_mlp(x, shards), eps)
    xin = oracle.layer_norm(x, eps) if layernorm else x
    Y = oracle.tp_mlp(xin, shards)
    return x + Y if residual else Y


def sample_rows(M: int, count: int, seed: int) -> np.ndarray:
    """Seeded row sample that always includes the first and last rows."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(count, M), replace=False).tolist())
    rows.update({0, M - 1})
    return np.array(sorted(rows), dtype=np.int64)


def sample_rows_per_tile(M: int, tile: int, seed: int) -> np.ndarray:
    """One seeded row from every `tile`-row block of M rows (the last block
    may be partial), plus the first and last rows."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1}
    for t0 in range(0, M, tile):
        rows.add(int(t0 + rng.integers(0, min(tile, M - t0))))
    return np.array(sorted(rows), dtype=np.int64)


__all__ = ["workloads", "oracle"]
