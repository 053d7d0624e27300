"""The gfx950 kernels as built (hipcc -S with the build's flags): no inline
assembly reads an MFMA result, an SGPR written by a VALU instruction, or M0
(the LDS address of an LDS-DMA load) before the wait states it needs (see
tests/asm_hazards.py).  A missing fence there reads stale values without any
error: the scores of a 16-pass fp8 MFMA were read 7 instructions after it
issued, and results differed from run to run; a buffer descriptor read 0
wait states after the v_readlane that wrote it gave a wrong d = 64 layer."""
import os
import shutil
import subprocess

import pytest

from static_triangle_sparse_amd import build as B
from tests.asm_hazards import find_hazards, find_sgpr_hazards

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
    out = tmp_path / (src + ".s")  # noqa: E501
    cmd = [hipcc, *B.HIPCC_FLAGS, "--cuda-device-only", "-S", "-I", B.INCLUDE, "-I", B.CSRC,
           os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:]
    return out.read_text()


@pytest.fixture(scope="module")
def assembly(hipcc, tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    return {src: _assembly(hipcc, src, d) for src in SOURCES}


@pytest.mark.parametrize("src", SOURCES)
def test_no_inline_asm_reads_fresh_mfma_results(assembly, src):
    hazards = find_hazards(assembly[src], NEED)
    assert not hazards, "\n".join(f"{k[:60]} line {ln}: {ins} ({d} wait states after MFMA at line {ml})"
                                  for k, ln, ins, ml, d in hazards[:10])


@pytest.mark.parametrize("src", SOURCES)
def test_no_inline_asm_memory_op_reads_a_fresh_sgpr_or_m0(assembly, src):
    text = assembly[src]
    hazards = find_sgpr_hazards(text)
    assert not hazards, "\n".join(f"{k[:60]} line {ln}: {ins} ({d} wait states after the {kind} write "
                                  f"at line {wl})" for k, ln, ins, wl, d, kind in hazards[:10])
    if src == "attn_fwd_gfx950.hip":
        # the scan saw the copies: LDS-DMA loads in inline assembly, each right
        # after a compiler-placed write of M0
        assert text.count("offen lds") >= 20


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


def _kernel(*lines):
    return "\n".join(["_Zkernel:", *lines])


def _asm(*lines):
    return [";;#ASMSTART", *lines, ";;#ASMEND"]


def test_the_sgpr_scan_finds_planted_hazards():
    load = "\tbuffer_load_dwordx4 v35, s[12:15], 0 offen lds"
    cases = {
        # a descriptor word from v_readfirstlane, read at once: hazard
        "readfirstlane": (_kernel("\tv_readfirstlane_b32 s14, v1", *_asm(load)), [("valu-sgpr", 0)]),
        # five wait states inside the asm block: enough
        "nop 4": (_kernel("\tv_readfirstlane_b32 s14, v1", *_asm("\ts_nop 4", load)), []),
        # four are not
        "nop 3": (_kernel("\tv_readlane_b32 s12, v1, 3", *_asm("\ts_nop 3", load)), [("valu-sgpr", 4)]),
        # a carry-out of a 64-bit multiply-add into the descriptor
        "carry": (_kernel("\tv_mad_u64_u32 v[36:37], s[12:13], v35, s8, v[36:37]", "\ts_add_u32 s2, s3, s4",
                          *_asm("\ts_nop 1", load)), [("valu-sgpr", 3)]),
        # an SGPR the load does not read: no hazard
        "other sgpr": (_kernel("\tv_readfirstlane_b32 s20, v1", *_asm(load)), []),
        # M0 written right before the LDS-DMA load: hazard; one wait state: enough
        "m0": (_kernel("\ts_mov_b32 m0, s80", *_asm(load)), [("m0", 0)]),
        "m0 nop": (_kernel("\ts_mov_b32 m0, s80", *_asm("\ts_nop 0", load)), []),
        # a load without lds does not read M0
        "m0 no lds": (_kernel("\ts_mov_b32 m0, s80", *_asm("\tbuffer_load_dwordx4 v[0:3], v35, s[12:15], 0 offen")),
                      []),
        # the write on the taken side of a branch reaches the load at the label
        "branch": (_kernel("\tv_readfirstlane_b32 s13, v1", "\ts_cbranch_scc1 .LBB0_2",
                           "\ts_nop 7", "\ts_nop 7", ".LBB0_2:", *_asm(load)), [("valu-sgpr", 1)]),
        # the compiler's own loads are its business (not inline assembly)
        "compiler load": (_kernel("\tv_readfirstlane_b32 s14, v1", load), []),
    }
    for name, (text, want) in cases.items():
        got = [(kind, d) for _, _, _, _, d, kind in find_sgpr_hazards(text)]
        assert got == want, (name, got)
