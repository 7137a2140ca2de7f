"""The large-block GEMM kernel issues its matrix-core operations from inline
asm without wait states, and the compiler cannot see into that asm: these
tests compile the GEMM source for gfx950 to assembly (no GPU needed) and check
the wait-state rules of asm_hazards on every path of that kernel, and that the
checker itself catches planted violations."""
import os
import shutil
import subprocess
import tempfile

import pytest

import asm_hazards
from quantized_gemm_qoq_amd import build as hipbuild


def _hipcc():
    try:
        return hipbuild.hipcc()
    except RuntimeError:
        return None


@pytest.fixture(scope="module")
def gemm_asm():
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    src = os.path.join(hipbuild.CSRC, "gemm.hip")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "gemm.s")
        flags = [f for f in hipbuild.common_flags() if f != "-fPIC"]
        cmd = [cc, *flags, "--cuda-device-only", "-S", src, "-o", out]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        assert proc.returncode == 0, proc.stderr[-2000:]
        with open(out) as f:
            return f.read()


def test_large_block_kernel_wait_states(gemm_asm):
    n, problems = asm_hazards.check(gemm_asm, "k_gemm_big")
    # 6 instantiations (3 weight formats x with/without the INT32 output),
    # 512 operations each in the unrolled group loop
    assert n >= 6 * 512
    assert problems == [], "\n".join(problems[:20])


_CLEAN = """\
k:
\tv_and_b32_e32 v4, 0xf0f0f0f, v9
\tds_read_b128 v[0:3], v10
\ts_nop 0
\ts_waitcnt lgkmcnt(0)
\tv_mfma_i32_16x16x64_i8 a[0:3], v[4:7], v[0:3], a[0:3]
\ts_nop 7
\ts_nop 1
\tv_accvgpr_read_b32 v20, a0
\ts_endpgm
"""


def test_checker_accepts_clean_sequence():
    n, problems = asm_hazards.check(_CLEAN, "k")
    assert n == 1 and problems == []


def test_checker_flags_valu_operand_write():
    bad = _CLEAN.replace("\ts_nop 0\n\ts_waitcnt lgkmcnt(0)\n", "")
    bad = bad.replace("\tds_read_b128 v[0:3], v10\n", "\tds_read_b128 v[0:3], v10\n\ts_waitcnt lgkmcnt(0)\n")
    # v_and writes v4, read as operand A 2 instructions later: fine; move it next to the op
    bad = bad.replace("\tv_and_b32_e32 v4, 0xf0f0f0f, v9\n", "")
    bad = bad.replace("\tv_mfma_i32", "\tv_and_b32_e32 v5, 0xf0f0f0f, v9\n\tv_mfma_i32", 1)
    n, problems = asm_hazards.check(bad, "k")
    assert n == 1 and len(problems) == 1 and "writes an operand" in problems[0]


def test_checker_flags_early_result_read():
    bad = _CLEAN.replace("\ts_nop 7\n\ts_nop 1\n", "\ts_nop 4\n")
    n, problems = asm_hazards.check(bad, "k")
    assert len(problems) == 1 and "5 wait states" in problems[0]


def test_checker_follows_branches():
    # the read is reached from a branch taken right after the operation
    text = """\
k:
\tv_mfma_i32_16x16x64_i8 a[0:3], v[4:7], v[0:3], a[0:3]
\ts_cbranch_scc1 .LBB0_2
\ts_nop 7
\ts_nop 7
.LBB0_2:
\tv_accvgpr_read_b32 v20, a1
\ts_endpgm
"""
    n, problems = asm_hazards.check(text, "k")
    assert len(problems) == 1 and "0 wait states" in problems[0]


def test_checker_reads_past_an_early_endpgm():
    # an early-exit path ends in s_endpgm before the rest of the function
    text = """\
k:
\ts_cbranch_scc1 .LBB0_9
\ts_endpgm
.LBB0_9:
\tv_mfma_i32_16x16x64_i8 a[0:3], v[4:7], v[0:3], a[0:3]
\tv_accvgpr_read_b32 v20, a1
\ts_endpgm
.Lfunc_end0:
"""
    n, problems = asm_hazards.check(text, "k")
    assert n == 1 and len(problems) == 1 and "0 wait states" in problems[0]
