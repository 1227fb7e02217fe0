"""The build's check of the MFMA GEMM's generated assembly (CPU only).

The check must flag an accumulator copy between the first MFMA and the
padding after the last one, and any scratch use; and the assembly of the
current build, when present, must pass it."""

import os

import pytest

from tensor_transformer_mlp_tpmlp_amd import build as B

KERNEL = "_ZN5tpmlp12_GLOBAL__N_114gemm_bf16_mfmaIXXXE"


def _asm(body_lines, scratch=0):
    body = "\n".join("\t" + l for l in body_lines)
    return (f"{KERNEL}:\n{body}\n.Lfunc_end0:\n\t; ScratchSize: {scratch}\n")


CLEAN = ["v_accvgpr_write_b32 a0, 0", "s_nop 7", "s_nop 7",
         "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]",
         "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[4:7], a[4:7]",
         "s_nop 7", "s_nop 7", "s_nop 7", "v_accvgpr_read_b32 v8, a0"]


def test_clean_kernel_passes():
    assert B.check_gemm_asm(_asm(CLEAN)) == []


def test_accumulator_copy_inside_the_mfma_region_is_flagged():
    bad = CLEAN[:4] + ["v_accvgpr_read_b32 v9, a1"] + CLEAN[4:]
    problems = B.check_gemm_asm(_asm(bad))
    assert len(problems) == 1 and "accumulator copy" in problems[0]


def test_read_hoisted_above_the_padding_is_flagged():
    bad = CLEAN[:5] + ["v_accvgpr_read_b32 v9, a4"] + CLEAN[5:]
    assert any("accumulator copy" in p for p in B.check_gemm_asm(_asm(bad)))


def test_scratch_is_flagged():
    assert any("scratch" in p for p in B.check_gemm_asm(_asm(CLEAN, scratch=36)))


def test_current_build_assembly_passes():
    path = os.path.join(B.BUILD_DIR, B.ASM_CHECKED + ".s")
    if not os.path.exists(path):
        pytest.skip("no assembly from a build in this tree")
    with open(path) as f:
        asm = f.read()
    assert asm.count("gemm_bf16_mfma") > 0
    assert B.check_gemm_asm(asm) == []
