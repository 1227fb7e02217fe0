#!/usr/bin/env python3
"""TP-MLP forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

NAME is a TP-MLP workload (default: the headline size), an attention
workload (attn_s{128,256,512}_bf16: the attention half of the block) or
block_s{128,256,512}_bf16 (the whole block with the time of each half).

One step is one full forward of the hot path, Y = sum_i GeLU_tanh(X A_i) B_i
(plus LayerNorm and the residual for the Post-LN workloads), over inputs
already resident in HBM.  Weights are packed before timing (they are static).
Prints ONE JSON line: whole-forward TFLOP/s (4*M*D*F per step, from the timed
loop), the roofline of the dominant kernel from HIP events recorded around
each kernel on a sample of the timed steps (live, inside the timed
region), and the fp64 oracle timed on the host cores on a row sample.
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
# Copy used to calibrate the byte counters: bf16 -> fp32 conversion of
# CALIB_ELEMS elements after the caches were flushed; it reads 2 and writes 4
# bytes per element (2 GiB read, 4 GiB written: far beyond the 256 MB
# Infinity Cache, so every byte crosses from the L2 to memory).
CALIB_ELEMS = 1 << 30
# What roofline.traffic measures: FETCH_SIZE and WRITE_SIZE count requests
# between the L2 and the fabric on one of the L2's memory interfaces; scaled
# by the calibration copy they estimate all bytes that leave the L2, which
# the Infinity Cache may serve in part (so they bound HBM traffic from above).
TRAFFIC_KIND = "bytes between L2 and the fabric (Infinity Cache or HBM), per launch"


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


def device_info() -> dict:
    """The GPU of the run: name, CU count and peak shader clock (HIP's
    hipDeviceAttributeClockRate, attribute 5, in kHz), and the dense bf16
    MFMA peak they give at 4096 FLOP per clock per CU (the 2516.6 TFLOP/s
    figure is 256 CUs at 2.4 GHz).  The clock the GEMMs sustain under load is
    lower; the counter profile of the headline GEMMs measures it."""
    import torch
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        khz = ctypes.c_int()
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, 0) == 0 and khz.value > 0:
            ghz = khz.value / 1e6
            info["peak_clock_ghz"] = round(ghz, 3)
            info["bf16_peak_tflops_from_cus_and_clock"] = round(props.multi_processor_count * 4096 * ghz / 1e3, 1)
    except OSError:
        pass
    return info


def _sha256(path: str) -> str:
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _traffic(workload: str, kernel: str, algorithmic_bytes: float):
    """Bytes between the L2 and the fabric per launch (TRAFFIC_KIND) from the
    committed rocprofv3 counter summary, if it was taken on the current kernel
    source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload, {}).get(kernel)
    if not entry or entry.get("source_sha256") != _sha256(KERNEL_SOURCES[kernel]):
        return None
    return entry.get("l2_fabric_bytes_per_launch")


def copy_calibration() -> None:
    """A plain copy of known size for calibrating FETCH_SIZE / WRITE_SIZE:
    flush the caches with 2 GiB of unrelated writes, then convert
    CALIB_ELEMS bf16 values (2 GiB read) to fp32 (4 GiB written)."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(CALIB_ELEMS, dtype=torch.bfloat16, device=dev)
    dst = torch.empty(CALIB_ELEMS, dtype=torch.float32, device=dev)
    flush = torch.empty(1 << 29, dtype=torch.float32, device=dev)
    flush.fill_(1.0)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst, flush
    log(f"[bench] copy calibration: {CALIB_ELEMS * 2 >> 20} MiB read, {CALIB_ELEMS * 4 >> 20} MiB written")


def summarize_profiles(trace_dir: str, fetch_dir: str, write_dir: str, workload: str, out_dir: str,
                       command: str, sq_dir: str = "") -> None:
    """Turn rocprofv3 CSV output (kernel trace + FETCH_SIZE + WRITE_SIZE runs of
    this bench) into the summaries kept under profiles/."""
    import csv
    import glob
    import statistics

    def rows(d, pattern):
        files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
        if not files:
            raise SystemExit(f"no {pattern} under {d}")
        with open(files[0]) as f:
            return list(csv.DictReader(f))

    def kind(name):
        if "gemm_bf16_mfma" in name:
            # gemm_bf16_mfma<Cfg<BM, BN, NU>, EPI, ...>: EPI 0 is GEMM1's GeLU epilogue
            epi = name.split("Cfg")[1].split("EEE", 1)[1]
            return "gemm1" if epi.startswith("Li0E") else "gemm2"
        if "copy" in name or "elementwise" in name:
            return "copy"
        return None

    stats = rows(trace_dir, "*kernel_stats.csv")
    trace = rows(trace_dir, "*kernel_trace.csv")
    durs = {}
    for r in trace:
        k = kind(r["Kernel_Name"])
        if k in ("gemm1", "gemm2"):
            durs.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def counter(d, name):
        per = {}
        for r in rows(d, "*counter_collection.csv"):
            if r["Counter_Name"] != name:
                continue
            per.setdefault((kind(r["Kernel_Name"]), r["Kernel_Name"], r["Dispatch_Id"]), 0.0)
            per[(kind(r["Kernel_Name"]), r["Kernel_Name"], r["Dispatch_Id"])] += float(r["Counter_Value"])
        return per

    fetch, write = counter(fetch_dir, "FETCH_SIZE"), counter(write_dir, "WRITE_SIZE")
    sq = {c: counter(sq_dir, c) for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "TCC_HIT_sum",
                                          "TCC_MISS_sum")} if sq_dir else {}

    def calib(per, expected_kib):
        vals = [v for (k, n, _), v in per.items() if k == "copy" and "bfloat16" in n and "float" in n]
        vals = [v for v in vals if v > expected_kib / 8]
        return expected_kib / max(vals) if vals else None

    f_read = calib(fetch, CALIB_ELEMS * 2 / 1024)
    f_write = calib(write, CALIB_ELEMS * 4 / 1024)
    with open(os.path.join(ROOT, KERNEL_SOURCES["gemm1"]), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    traffic = {}
    lines = [f"# rocprofv3 summary: TP-MLP forward, workload {workload}", "",
             f"command (kernel trace): {command}", "", "## kernel trace (average over dispatches)", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for k in ("gemm1", "gemm2"):
        d = durs.get(k, [])
        if d:
            lines.append(f"| {k} | {len(d)} | {statistics.mean(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
    lines += ["", "all kernels (rocprofv3 --stats):", "", "| name | calls | average ns |", "|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['Name'][:110]} | {r['Calls']} | {float(r['AverageNs']):.0f} |")
    if sq:
        import statistics as st

        def mean_of(c, k):
            v = [x for (kk, _, _), x in sq[c].items() if kk == k]
            return st.mean(v) if v else None
        lines += ["", "## MFMA busy, clock and L2 hit rate (rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES "
                  "GRBM_GUI_ACTIVE TCC_HIT_sum TCC_MISS_sum)", "",
                  "GRBM_GUI_ACTIVE is summed over the 8 XCDs, so GRBM_GUI_ACTIVE / 8 is the kernel's length in "
                  "shader cycles and GRBM_GUI_ACTIVE / 8 / duration its average clock.  MFMA busy = "
                  "SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs) / (1024 GRBM_GUI_ACTIVE / 8): the "
                  "fraction of SIMD cycles in which the matrix core was busy.", "",
                  "| kernel | SQ_VALU_MFMA_BUSY_CYCLES | GRBM_GUI_ACTIVE | clock GHz (trace duration) | MFMA busy "
                  "| L2 hit rate |", "|---|---|---|---|---|---|"]
        for k in ("gemm1", "gemm2"):
            busy, act = mean_of("SQ_VALU_MFMA_BUSY_CYCLES", k), mean_of("GRBM_GUI_ACTIVE", k)
            hit, miss = mean_of("TCC_HIT_sum", k), mean_of("TCC_MISS_sum", k)
            d = durs.get(k)
            if busy and act and d:
                cyc = act / 8
                lines.append(f"| {k} | {busy:.4g} | {act:.4g} | {cyc / (st.mean(d) * 1e3):.2f} | "
                             f"{busy / (1024 * cyc):.3f} | {hit / (hit + miss):.3f} |")
    lines += ["", "## Bytes between the L2 and the fabric (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE; "
              "KiB per dispatch)", "",
              "FETCH_SIZE and WRITE_SIZE count requests on one of the L2's memory interfaces; they are scaled by "
              "what they read for the calibration copy.  The bytes leave the L2; the 256 MB Infinity Cache may "
              "serve part of them, so they bound HBM traffic from above.", "",
              f"calibration copy: {CALIB_ELEMS * 2 >> 20} MiB read / {CALIB_ELEMS * 4 >> 20} MiB written; "
              f"scale factors read {f_read}, write {f_write}", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes per launch (L2 <-> fabric) |", "|---|---|---|---|"]
    for k in ("gemm1", "gemm2"):
        fv = [v for (kk, _, _), v in fetch.items() if kk == k]
        wv = [v for (kk, _, _), v in write.items() if kk == k]
        if fv and wv and f_read and f_write:
            b = (statistics.mean(fv) * f_read + statistics.mean(wv) * f_write) * 1024
            traffic[k] = {"fetch_kib": statistics.mean(fv), "write_kib": statistics.mean(wv),
                          "l2_fabric_bytes_per_launch": b, "kind": TRAFFIC_KIND, "source_sha256": sha}
            lines.append(f"| {k} | {statistics.mean(fv):.0f} | {statistics.mean(wv):.0f} | {b:.4g} |")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"tpmlp_forward_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    try:
        with open(TRAFFIC_FILE) as f:
            allt = json.load(f)
    except (OSError, ValueError):
        allt = {}
    allt[workload] = {"read_scale": f_read, "write_scale": f_write, **traffic}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allt, f, indent=1)
    print("\n".join(lines))


def host_description() -> str:
    """CPU model and BLAS library of the host, for the oracle baseline."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas = f"{p.get('internal_api', 'blas')} {p.get('version', '')}".strip()
                break
    except Exception:
        pass
    return f"{model}; {blas}"


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
        elif w.layernorm_after:
            oracle.norm_after_ffn(x, shards)
        else:
            oracle.tp_mlp(x, shards)
        return time.perf_counter() - t0

    # size the sample from a 64-row probe: the whole workload when it fits the
    # target time, else a row prefix of about that length
    probe = min(64, w.M)
    run(min(16, w.M))  # warm the BLAS thread pool and the allocator first
    t_probe = run(probe)
    est_full = t_probe * w.M / probe
    rows = w.M if est_full <= target_s else int(max(probe, w.M * target_s / est_full))
    t = run(rows)
    flops = 4.0 * rows * w.D * w.F
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"all {w.M} rows" if rows == w.M else f"first {rows} of {w.M} rows of X (rows are "
                       "independent)") + f", D={w.D}, F={w.F}, n={w.n}; numpy fp64 oracle, {t:.1f} s; "
                      + host_description()}


BWD_METRIC = "TP-MLP backward TFLOP/s (8·M·D·F: dX, dA, dB), 1 MI355X"


def bench_backward(args, w, inp, X, shards, dtype, dev) -> int:
    """Times tpmlp_backward: gradients dX, dA, dB for a seeded bf16 dY.

    value = 8·M·D·F / t, the algorithmic FLOP of the four gradient GEMMs.
    As in a training step, the forward (run once, untimed) keeps the
    pre-activation S = X A and the activation H = GeLU(S), so the backward
    recomputes neither.  The events bracket the whole pass on the library's
    stream.
    """
    import numpy as np
    import torch

    import tensor_transformer_mlp_tpmlp_amd as tp
    import workloads

    if w.layernorm or w.residual or w.layernorm_after:
        raise SystemExit("the backward covers the TP-MLP without LayerNorm or residual")
    dYh = np.random.default_rng(w.seed + 7).standard_normal((w.M, w.D)).astype(np.float32)
    if w.dtype == "bf16":
        dYh = workloads.round_to_bf16(dYh)
    dY = torch.from_numpy(dYh).to(dev).to(dtype).contiguous()
    outs = (torch.empty_like(X), torch.empty((w.D, w.F), dtype=dtype, device=dev),
            torch.empty((w.F, w.D), dtype=dtype, device=dev))
    # the forward of a training step keeps the pre-activation and the
    # activation for the backward
    S = torch.empty((w.M, w.F), dtype=dtype, device=dev)
    H = torch.empty((w.M, w.F), dtype=dtype, device=dev)
    tp.tp_mlp(X, shards, save_preact=S, save_act=H)

    def step():
        tp.tp_mlp_backward(X, dY, shards, out=outs, preact=S, act=H)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    log(f"[bench] backward: {args.steps} timed steps, {ms:.4f} ms/step")
    flops = 8.0 * w.M * w.D * w.F
    value = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    out = {
        "metric": BWD_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "strong", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward", "M": w.M, "D": w.D, "F": w.F, "n": w.n},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "kernel": "whole backward pass", "achieved": round(value, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(value / peak, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle
        log("[bench] timing the fp64 oracle backward on the host")
        cores = len(os.sched_getaffinity(0))

        def run(rows):
            t = time.perf_counter()
            oracle.tp_mlp_backward_full(inp.X[:rows], inp.A, inp.B, w.n, dYh[:rows])
            return time.perf_counter() - t

        run(min(16, w.M))
        probe = min(64, w.M)
        t_probe = run(probe)
        rows = w.M if t_probe * w.M / probe <= args.cpu_seconds else max(probe, int(probe * args.cpu_seconds / t_probe))
        rows = min(rows, w.M)
        t_cpu = run(rows)
        out["cpu_baseline"] = {
            "value": 8.0 * rows * w.D * w.F / t_cpu / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"{'all' if rows == w.M else 'first'} {rows} of {w.M} rows of X and dY, D={w.D}, F={w.F}, "
                       f"n={w.n}; numpy fp64 oracle backward (S, H, dS, dX, dA, dB), {t_cpu:.1f} s; the weight "
                       "gradients over a row prefix cost the same per row as over all rows"),
        }
    print(json.dumps(out), flush=True)
    return 0


ATTN_METRIC = "attention half TFLOP/s (2·M·h·3h projection + 4·b·s²·h scores and P·V), 1 MI355X"
BLOCK_METRIC = "block forward ms per step (attention half + FFN half), 1 MI355X"


def _timed_segments(args, step, nev, warm=True):
    """Warm up, then time args.steps calls of step(events) between two events
    on the stream.  One timed step in `every` (every = max(4, steps / 10),
    so about ten samples) also records nev HIP events around its kernels
    (the library's event argument), so the per-kernel intervals are measured
    live, inside the timed region; the other steps pass none, which keeps
    the records' few microseconds of queue time out of most steps (it
    matters only for steps of tens of microseconds).  Returns (ms per step,
    [mean ms of each of the nev - 1 intervals over the sampled steps])."""
    import numpy as np
    import torch

    every = max(4, args.steps // 10)

    if warm:
        for _ in range(args.warmup):
            step(None)
    torch.cuda.synchronize()
    hip = HipEvents()
    sampled = [k for k in range(args.steps) if k % every == every - 1] or [args.steps - 1]
    evs = {k: [hip.create() for _ in range(nev)] for k in sampled}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(args.steps):
        step(evs.get(k))
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    seg = [float(np.mean([hip.elapsed_ms(e[i], e[i + 1]) for e in evs.values()])) for i in range(nev - 1)]
    whole = [hip.elapsed_ms(e[0], e[nev - 1]) for e in evs.values()]
    hip.close()
    _timed_segments.step_stats = {"min": float(np.min(whole)), "median": float(np.median(whole)),
                                  "sampled_steps": len(whole)}
    return ms, seg


def _oracle_cores() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"),
                       default=os.cpu_count()))
    except Exception:
        return int(os.cpu_count() or 1)


def bench_attention(args, w) -> int:
    """The attention half (LayerNorm, QKV projection, per-head softmax
    attention, heads concatenated, residual) on one attention workload."""
    import numpy as np
    import torch

    import tensor_transformer_mlp_tpmlp_amd as tp
    import workloads

    dev = torch.device("cuda:0")
    inp = workloads.make_attn_inputs(w)
    x, Wq, Wk, Wv = (torch.from_numpy(a).to(dev).to(torch.bfloat16).contiguous()
                     for a in (inp.x, inp.Wq, inp.Wk, inp.Wv))
    aw = tp.shard_attention(Wq, Wk, Wv, w.heads, w.p)
    out = torch.empty_like(x)
    torch.cuda.synchronize()

    def step(ev):
        tp.attention(x, w.batch, w.seq, aw, out=out, events=ev)

    ms, (t_ln, t_proj, t_attn) = _timed_segments(args, step, 4)
    log(f"[bench] {w.name}: {ms:.4f} ms/step (LN {t_ln:.4f}, projection {t_proj:.4f}, attention {t_attn:.4f})")
    value = w.flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16"]
    f_proj = 2.0 * w.M * w.hidden * 3 * w.hidden
    f_attn = 4.0 * w.batch * w.seq * w.seq * w.hidden
    kernel, t_k, f_k = ("attention", t_attn, f_attn) if t_attn >= t_proj else ("qkv_projection", t_proj, f_proj)
    achieved = f_k / (t_k * 1e-3) / 1e12
    res = {
        "metric": ATTN_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "strong", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq": w.seq, "hidden": w.hidden, "heads": w.heads,
                   "p": w.p, "layernorm": True, "residual": True, "out_proj": False},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "kernels_ms": {"ln_stats": round(t_ln, 5), "qkv_projection": round(t_proj, 5),
                       "attention": round(t_attn, 5)},
        "roofline": {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        from oracle import attention_oracle as ao
        log("[bench] timing the fp64 oracle on the host")

        def run(nb):
            t0 = time.perf_counter()
            ao.attention_half(inp.x[:nb * w.seq], inp.Wq, inp.Wk, inp.Wv, w.heads, w.p, nb, w.seq)
            return time.perf_counter() - t0

        run(1)
        t1 = run(1)
        nb = max(1, min(w.batch, int(args.cpu_seconds / max(t1, 1e-6))))
        t = run(nb)
        res["cpu_baseline"] = {
            "value": w.flops * nb / w.batch / t / 1e12, "unit": "TFLOP/s", "cores": _oracle_cores(),
            "kind": "oracle",
            "sample": f"{'all' if nb == w.batch else 'first'} {nb} of {w.batch} sequences (independent), "
                      f"s={w.seq}, h={w.hidden}, {w.heads} heads; numpy fp64 oracle, {t:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


def bench_block(args, s: int) -> int:
    """The block forward of "LLM Lab Notes 06" (code order): x1 = x +
    attn(LayerNorm(x)), out = x1 + TP-MLP(LayerNorm(x1)), with the time of
    each half (the page's segment timing)."""
    import torch

    import tensor_transformer_mlp_tpmlp_amd as tp
    import workloads

    wa = workloads.ATTN_WORKLOADS[f"attn_s{s}_bf16"]
    wf = workloads.WORKLOADS[f"postln_s{s}_bf16"]
    dev = torch.device("cuda:0")
    ai = workloads.make_attn_inputs(wa)
    fi = workloads.make_inputs(wf)
    bf = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16).contiguous()
    x = bf(ai.x)
    aw = tp.shard_attention(bf(ai.Wq), bf(ai.Wk), bf(ai.Wv), wa.heads, wa.p)
    shards = tp.shard_mlp(bf(fi.A), bf(fi.B), wf.n)
    x1, y = torch.empty_like(x), torch.empty_like(x)
    torch.cuda.synchronize()

    def step(ev):
        tp.block(x, wa.batch, wa.seq, aw, shards, x1=x1, out=y, events=ev)

    ms, (t_attn, t_ffn) = _timed_segments(args, step, 3)
    log(f"[bench] block s={s}: {ms:.4f} ms/step (attention {t_attn:.4f}, FFN {t_ffn:.4f})")
    flops = wa.flops + wf.flops
    res = {
        "metric": BLOCK_METRIC, "value": round(ms, 5), "unit": "ms", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": False, "scaling": "strong", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"block_s{s}_bf16", "batch": wa.batch, "seq": s, "hidden": wa.hidden,
                   "heads": wa.heads, "ffn": wf.F, "p": wa.p},
        "segments_ms": {"attention": round(t_attn, 5), "ffn": round(t_ffn, 5)},
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
    }
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline bf16 size)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run the plain copy used to calibrate the HBM byte counters first")
    ap.add_argument("--summarize-profiles", nargs="+", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 CSV output of this bench: TRACE_DIR FETCH_DIR "
                         "WRITE_DIR [SQ_DIR] (SQ_DIR: SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE TCC_HIT_sum "
                         "TCC_MISS_sum)")
    ap.add_argument("--profile-command", default="", help="command recorded in the profile summary")
    ap.add_argument("--pass", dest="which", choices=("forward", "backward"), default="forward",
                    help="time the forward (default, the headline metric) or the backward pass")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")

    if args.summarize_profiles:
        import workloads
        d = args.summarize_profiles
        if len(d) not in (3, 4):
            ap.error("--summarize-profiles takes TRACE_DIR FETCH_DIR WRITE_DIR [SQ_DIR]")
        summarize_profiles(d[0], d[1], d[2], args.workload or workloads.HEADLINE,
                           os.path.join(ROOT, "profiles"), args.profile_command, d[3] if len(d) == 4 else "")
        return 0

    if args.gpus != 1:
        msg = (f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
               "(the multi-GPU all-reduce is not implemented; the one-GPU path sums the shards on-chip)")
        print(msg, file=sys.stderr)
        print(json.dumps({"error": msg, "n_gpus": args.gpus}))
        return 2

    import numpy as np
    import torch

    import tensor_transformer_mlp_tpmlp_amd as tp
    import workloads

    name = args.workload or workloads.HEADLINE
    if name in workloads.ATTN_WORKLOADS:
        return bench_attention(args, workloads.ATTN_WORKLOADS[name])
    if name.startswith("block_s"):
        return bench_block(args, int(name[len("block_s"):].split("_")[0]))
    w = workloads.WORKLOADS[name]
    if args.copy_calibration:
        copy_calibration()
    dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    log(f"[bench] workload {w.name}: M={w.M} D={w.D} F={w.F} n={w.n} {w.dtype} "
        f"layernorm={w.layernorm} residual={w.residual} layernorm_after={w.layernorm_after}")
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
    if args.which == "backward":
        return bench_backward(args, w, inp, X, shards, dtype, dev)

    def step(events=None):
        tp.tp_mlp(X, shards, layernorm=w.layernorm, layernorm_after=w.layernorm_after, residual=residual,
                  out=Y, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")

    ms, (t_ln, t_g1, t_g2) = _timed_segments(args, step, 4, warm=False)
    t_ln, t_g1, t_g2 = [t_ln], [t_g1], [t_g2]
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
    if roofline["traffic"] is not None:
        roofline["traffic_kind"] = TRAFFIC_KIND
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "strong", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "D": w.D, "F": w.F, "n": w.n,
                   "layernorm": w.layernorm, "residual": w.residual, "layernorm_after": w.layernorm_after},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "step_ms_instrumented": {k: round(v, 5) for k, v in _timed_segments.step_stats.items()},
        "kernels_ms": {"ln_stats": round(float(np.mean(t_ln)), 5), "gemm1_gelu": round(g1, 5),
                       ("gemm2_sum_and_layernorm" if w.layernorm_after else "gemm2_sum"): round(g2, 5)},
        "roofline": roofline,
        "device": device_info(),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
