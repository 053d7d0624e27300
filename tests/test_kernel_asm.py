"""The gfx950 kernels as built (hipcc -S with the build's flags): no inline
assembly reads an MFMA result before the wait states it needs (see
tests/asm_hazards.py).  A missing fence there reads stale accumulators
without any error: the scores of a 16-pass fp8 MFMA were read 7
instructions after it issued, and results differed from run to run."""
import os
import shutil
import subprocess

import pytest

from static_triangle_sparse_amd import build as B
from tests.asm_hazards import find_hazards

# an MFMA of 16 passes needs 18 wait states before a VALU read (2 + passes);
# one more for margin
NEED = 19
SOURCES = ["attn_fwd_gfx950.hip", "dyn_select_gfx950.hip", "tiers_gfx950.hip", "split_gfx950.hip"]


@pytest.fixture(scope="module")
def hipcc():
    path = os.path.join(B.ROCM, "bin", "hipcc")
    if not os.path.exists(path) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    return path if os.path.exists(path) else shutil.which("hipcc")


def _assembly(hipcc, src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [hipcc, *B.HIPCC_FLAGS, "--cuda-device-only", "-S", "-I", B.INCLUDE, "-I", B.CSRC,
           os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:]
    return out.read_text()


@pytest.mark.parametrize("src", SOURCES)
def test_no_inline_asm_reads_fresh_mfma_results(hipcc, src, tmp_path):
    text = _assembly(hipcc, src, tmp_path)
    hazards = find_hazards(text, NEED)
    assert not hazards, "\n".join(f"{k[:60]} line {ln}: {ins} ({d} wait states after MFMA at line {ml})"
                                  for k, ln, ins, ml, d in hazards[:10])


def test_the_scan_finds_a_planted_hazard():
    # a synthetic kernel: an MFMA, two instructions, an inline-asm read of its
    # result (hazard); a fenced read (no hazard); a read behind a branch whose
    # taken path is short (hazard)
    asm = "\n".join([
        "_Zkernel:",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
        "\tv_add_u32 v30, v31, v32",
        ";;#ASMSTART", "\tv_max3_f32 v40, v0, v1, v2", ";;#ASMEND",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
        ";;#ASMSTART", "\ts_nop 7\n\ts_nop 7\n\ts_nop 4", ";;#ASMEND",
        ";;#ASMSTART", "\tv_max3_f32 v41, v0, v1, v2", ";;#ASMEND",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
        "\ts_cbranch_scc1 .LBB0_2",
        "\ts_nop 7", "\ts_nop 7", "\ts_nop 7",
        ".LBB0_2:",
        ";;#ASMSTART", "\tv_bfi_b32 v3, v42, s0, v3", ";;#ASMEND",
    ])
    got = [(ins.split()[0], d) for _, _, ins, _, d in find_hazards(asm, NEED)]
    assert got == [("v_max3_f32", 1), ("v_bfi_b32", 1)]
