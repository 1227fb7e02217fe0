#!/usr/bin/env python3
"""TP-MLP forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one full forward of the hot path, Y = sum_i GeLU_tanh(X A_i) B_i
(plus LayerNorm and the residual for the Post-LN workloads), over inputs
already resident in HBM.  Weights are packed before timing (they are static).
Prints ONE JSON line: whole-forward TFLOP/s (4*M*D*F per step), the roofline
of the dominant kernel from HIP events recorded around each kernel inside the
timed loop, and the fp64 oracle timed on the host cores on a row sample.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TP-MLP forward TFLOP/s (4·M·D·F) and % of bf16 MFMA peak, 1 MI355X"
# MI355X dense matrix-core peaks (no sparsity): 256 CUs at 2.4 GHz.
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
KERNEL_SOURCES = {"gemm1": "tensor_transformer_mlp_tpmlp_amd/csrc/gemm_bf16.hip",
                  "gemm2": "tensor_transformer_mlp_tpmlp_amd/csrc/gemm_bf16.hip"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles via the HIP runtime (timing on the library's stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def create(self) -> int:
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.events.append(e.value)
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def _sha256(path: str) -> str:
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _traffic(workload: str, kernel: str, algorithmic_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload, {}).get(kernel)
    if not entry or entry.get("source_sha256") != _sha256(KERNEL_SOURCES[kernel]):
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, target_s: float):
    """The fp64 oracle, untuned, on a bounded row sample of the same workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"),
                      default=os.cpu_count())
    except Exception:
        threads = os.cpu_count()
    shards = oracle.shard_mlp(inp.A.astype(np.float64), inp.B.astype(np.float64), w.n)
    X = inp.X.astype(np.float64)

    def run(rows):
        x = X[:rows]
        t0 = time.perf_counter()
        if w.layernorm:
            oracle.post_ln_ffn(x, shards)
        else:
            oracle.tp_mlp(x, shards)
        return time.perf_counter() - t0

    probe = min(8, w.M)
    t_probe = run(probe)
    rows = int(min(w.M, max(probe, probe * target_s / max(t_probe, 1e-6))))
    t = run(rows)
    flops = 4.0 * rows * w.D * w.F
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {rows} of {w.M} rows of X (rows are independent), full D={w.D}, F={w.F}, "
                      f"n={w.n}; numpy fp64, {t:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline bf16 size)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        msg = (f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
               "(the multi-GPU all-reduce is not part of this build)")
        print(msg, file=sys.stderr)
        print(json.dumps({"error": msg, "n_gpus": args.gpus}))
        return 2

    import numpy as np
    import torch

    import tensor_transformer_mlp_tpmlp_amd as tp
    import workloads

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    log(f"[bench] workload {w.name}: M={w.M} D={w.D} F={w.F} n={w.n} {w.dtype} "
        f"layernorm={w.layernorm} residual={w.residual}")
    t0 = time.time()
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    X, A, B = (torch.from_numpy(a).to(dev).to(dtype).contiguous() for a in (inp.X, inp.A, inp.B))
    shards = tp.shard_mlp(A, B, w.n)
    del A, B
    residual = X if w.residual else None
    Y = torch.empty((w.M, w.D), dtype=dtype, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s")

    def step(events=None):
        tp.tp_mlp(X, shards, layernorm=w.layernorm, residual=residual, out=Y, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")

    hip = HipEvents()
    evs = [[hip.create() for _ in range(4)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(evs[k])
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    t_ln = [hip.elapsed_ms(e[0], e[1]) for e in evs]
    t_g1 = [hip.elapsed_ms(e[1], e[2]) for e in evs]
    t_g2 = [hip.elapsed_ms(e[2], e[3]) for e in evs]
    hip.close()
    log(f"[bench] {args.steps} timed steps: {ms:.4f} ms/step")

    flops = float(w.flops)
    value = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    g1, g2 = float(np.mean(t_g1)), float(np.mean(t_g2))
    kernel, t_k = ("gemm1", g1) if g1 >= g2 else ("gemm2", g2)
    achieved = (2.0 * w.M * w.D * w.F) / (t_k * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": _traffic(w.name, kernel, 0.0)}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "strong", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "D": w.D, "F": w.F, "n": w.n,
                   "layernorm": w.layernorm, "residual": w.residual},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "kernels_ms": {"ln_stats": round(float(np.mean(t_ln)), 5), "gemm1_gelu": round(g1, 5),
                       "gemm2_sum": round(g2, 5)},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
