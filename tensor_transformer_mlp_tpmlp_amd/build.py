"""Build libtpmlp.so for gfx950 with hipcc, in-tree.

    python -m tensor_transformer_mlp_tpmlp_amd.build

Compiles every source under csrc/ to an object in _build/ (in parallel) and
links them into tensor_transformer_mlp_tpmlp_amd/libtpmlp.so.  hipcc
cross-compiles for gfx950 without a GPU present.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libtpmlp.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["tpmlp_api.cpp", "attention_api.cpp", "elementwise.hip", "gemm_generic.hip", "gemm_bf16.hip",
           "attention.hip", "noalloc.hip"]

# -packed-fp32-ops: never emit packed fp32 VALU instructions (v_pk_*_f32).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Per-file options.  attention.hip: MFMA results in VGPRs (the softmax reads
# and rescales them every tile; in AGPRs each access would need a copy), and
# the floating-point mode without IEEE NaN quieting, so that a maximum is one
# v_max_f32 rather than two operands quieted first (a third of the kernel's
# maxima were quieting operations); NaN inputs to the attention half give
# unspecified results.
EXTRA_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


# The throughput GEMM issues its MFMAs as inline assembly with the
# accumulators tied to AGPRs, so the compiler neither tracks their latency
# nor pads its own instructions against them.  Any accumulator copy the
# register allocator inserts between the first MFMA and the padding after
# the last one could read a stale value, and any spill would sit in the K
# loop.  Both depend on register-allocation choices, so every build checks
# the generated assembly of every instantiation of that kernel.
ASM_CHECKED = "gemm_bf16.hip"
_GEMM_KERNEL = re.compile(r"^(_ZN5tpmlp\S*gemm_bf16_mfma\S*):", re.M)


def check_gemm_asm(asm: str) -> list:
    """Problems in the assembly of the MFMA GEMM kernels (empty if none)."""
    problems = []
    for m in _GEMM_KERNEL.finditer(asm):
        name = m.group(1)
        end = asm.index(".Lfunc_end", m.end())
        body = asm[m.end():end].split("\n")
        meta = asm[end:end + 4000]
        scratch = re.search(r"; ScratchSize: (\d+)", meta)
        if scratch and int(scratch.group(1)) != 0:
            problems.append(f"{name}: {scratch.group(1)} bytes of scratch (spills)")
        mfma = [k for k, l in enumerate(body) if "v_mfma" in l]
        pad = [k for k, l in enumerate(body) if l.strip() == "s_nop 7"]
        if not mfma or len(pad) < 3:
            problems.append(f"{name}: no MFMA or no padding found")
            continue
        for k in range(mfma[0], pad[-3]):
            if re.search(r"v_accvgpr_(read|write|mov)", body[k]):
                problems.append(f"{name}: accumulator copy inside the MFMA region: {body[k].strip()}")
                break
    return problems


def _asm_check() -> None:
    asm_path = os.path.join(BUILD_DIR, ASM_CHECKED + ".s")
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, "--cuda-device-only", "-S", "-x", "hip",
           os.path.join(CSRC, ASM_CHECKED), "-o", asm_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {ASM_CHECKED}:\n{res.stderr}")
    with open(asm_path) as f:
        problems = check_gemm_asm(f.read())
    if problems:
        raise RuntimeError("the MFMA GEMM's register allocation is unsafe:\n" + "\n".join(problems))


def build(verbose: bool = True) -> str:
    """Compile all sources and link libtpmlp.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        check = ex.submit(_asm_check)
        objs = list(ex.map(_compile, SOURCES))
        check.result()
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()
