"""Static check of built gfx950 assembly: inline-assembly instructions that
read a VGPR written by an MFMA fewer than `need` wait states earlier.

The compiler inserts the wait states an MFMA result needs before its own
VALU instructions, but it does not look inside inline assembly; a helper
written in assembly that reads a fresh MFMA result must provide them
itself.  The scan follows each kernel forward, carries the pending MFMA
writes to the target label of every branch (keeping the shortest distance
over the incoming paths), ignores back edges (a loop body is longer than the
window), and counts s_nop n as n + 1 wait states and any other instruction
as one.  A newer MFMA writing the same registers replaces the older write.
"""
from __future__ import annotations

import re

_LABEL = re.compile(r"^(\.LBB\w+):")
_KERNEL = re.compile(r"^(_Z\S+):")


def _vregs(tok: str) -> frozenset:
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return frozenset({int(m.group(1))}) if m else frozenset()


def _merge(a: dict, b: dict) -> dict:
    out = dict(a)
    for regs, (dist, line) in b.items():
        if regs not in out or dist < out[regs][0]:
            out[regs] = (dist, line)
    return out


def find_hazards(asm_text: str, need: int):
    """[(kernel, line, instruction, mfma_line, wait_states)] of every hazard."""
    found = []
    kernel = None
    in_asm = False
    pending: dict = {}   # destination registers -> (wait states since, line)
    at_label: dict = {}
    dead = False
    for no, raw in enumerate(asm_text.splitlines(), 1):
        m = _KERNEL.match(raw)
        if m:
            kernel, pending, at_label, dead = m.group(1), {}, {}, False
            continue
        if kernel is None:
            continue
        s = raw.strip()
        m = _LABEL.match(s)
        if m:
            pending = _merge({} if dead else pending, at_label.pop(m.group(1), {}))
            dead = False
            continue
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith((".", ";")) or s.endswith(":"):
            continue
        parts = [t.strip(",") for t in s.split()]
        op, args = parts[0], parts[1:]
        if in_asm and args:
            reads = frozenset().union(*(_vregs(t) for t in args[1:])) if len(args) > 1 else frozenset()
            for regs, (dist, line) in pending.items():
                if reads & regs and dist < need:
                    found.append((kernel, no, s, line, dist))
        step = int(args[0]) + 1 if op == "s_nop" else 1
        pending = {r: (d + step, l) for r, (d, l) in pending.items() if d + step < 4 * need}
        if op.startswith("v_mfma"):
            dst = _vregs(args[0])
            pending = {r: v for r, v in pending.items() if not r <= dst}
            pending[dst] = (0, no)
        if op.startswith("s_cbranch") or op == "s_branch":
            at_label[args[0]] = _merge(at_label.get(args[0], {}), pending)
            dead = op == "s_branch"
    return found


# ---------------------------------------------------------------- SGPR / M0
#
# Two more wait-state rules that inline assembly must honour itself (the
# compiler's hazard recognizer does not look into it), from the CDNA3/CDNA4
# instruction-set documentation's table of manually inserted wait states:
#   * a VALU instruction that writes an SGPR (v_readlane, v_readfirstlane,
#     a VOP3 compare or a carry-out) followed by a memory instruction that
#     reads that SGPR (a buffer descriptor, an offset): 5 wait states;
#   * a write of M0 followed by an LDS-DMA load (buffer_load ... lds, which
#     takes its LDS address from M0): 1 wait state.
# The scan follows each kernel as find_hazards does and reports inline-asm
# memory instructions that are too close to such a write.

VALU_SGPR_NEED = 5
M0_LDS_NEED = 1

_SREG = re.compile(r"^s\[(\d+):(\d+)\]$|^s(\d+)$")
_SPECIAL = {"vcc": (106, 107), "vcc_lo": (106,), "vcc_hi": (107,)}


def _sregs(tok: str) -> frozenset:
    tok = tok.strip(",")
    if tok in _SPECIAL:
        return frozenset(_SPECIAL[tok])
    m = _SREG.match(tok)
    if not m:
        return frozenset()
    if m.group(3) is not None:
        return frozenset({int(m.group(3))})
    return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))


def _valu_sgpr_writes(op: str, args) -> frozenset:
    """SGPRs a VALU instruction writes: an SGPR destination (readlane,
    readfirstlane, VOP3 compares), or the carry-out of the 64-bit multiply-add
    and carry forms (second operand), or VCC of a VOPC compare."""
    if not op.startswith("v_") or not args:
        return frozenset()
    out = _sregs(args[0])
    if len(args) > 1 and (op.startswith(("v_mad_u64_u32", "v_mad_i64_i32", "v_div_scale"))
                          or "_co_" in op):
        out |= _sregs(args[1])
    if op.startswith("v_cmp") and op.endswith("_e32"):
        out |= frozenset(_SPECIAL["vcc"])
    return out


def _is_vmem(op: str) -> bool:
    return op.startswith(("buffer_", "global_", "scratch_", "flat_"))


def find_sgpr_hazards(asm_text: str, valu_need: int = VALU_SGPR_NEED, m0_need: int = M0_LDS_NEED):
    """[(kernel, line, instruction, writer_line, wait_states, kind)] of every
    inline-asm memory instruction that reads an SGPR fewer than `valu_need`
    wait states after a VALU write of it (kind "valu-sgpr"), or is an LDS-DMA
    load fewer than `m0_need` wait states after a write of M0 (kind "m0")."""
    found = []
    kernel = None
    in_asm = False
    pending: dict = {}   # ("s", reg) or ("m0",) -> (wait states since the write, line)
    at_label: dict = {}
    dead = False
    horizon = max(valu_need, m0_need) + 1

    def merge(a, b):
        out = dict(a)
        for key, (dist, line) in b.items():
            if key not in out or dist < out[key][0]:
                out[key] = (dist, line)
        return out

    for no, raw in enumerate(asm_text.splitlines(), 1):
        m = _KERNEL.match(raw)
        if m:
            kernel, pending, at_label, dead = m.group(1), {}, {}, False
            continue
        if kernel is None:
            continue
        s = raw.strip()
        m = _LABEL.match(s)
        if m:
            pending = merge({} if dead else pending, at_label.pop(m.group(1), {}))
            dead = False
            continue
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith((".", ";")) or s.endswith(":"):
            continue
        parts = [t.strip(",") for t in s.split()]
        op, args = parts[0], parts[1:]
        if in_asm and _is_vmem(op):
            reads = frozenset().union(*(_sregs(t) for t in args)) if args else frozenset()
            for key, (dist, line) in pending.items():
                if key[0] == "s" and key[1] in reads and dist < valu_need:
                    found.append((kernel, no, s, line, dist, "valu-sgpr"))
                if key == ("m0",) and "lds" in args and dist < m0_need:
                    found.append((kernel, no, s, line, dist, "m0"))
        step = int(args[0]) + 1 if op == "s_nop" else 1
        pending = {k: (d + step, l) for k, (d, l) in pending.items() if d + step < horizon}
        for r in _valu_sgpr_writes(op, args):
            pending[("s", r)] = (0, no)
        if args and args[0] == "m0":
            pending[("m0",)] = (0, no)
        if op.startswith("s_cbranch") or op == "s_branch":
            at_label[args[0]] = merge(at_label.get(args[0], {}), pending)
            dead = op == "s_branch"
    # one report per (line, kind)
    seen, out = set(), []
    for f in found:
        if (f[1], f[5]) not in seen:
            seen.add((f[1], f[5]))
            out.append(f)
    return out
