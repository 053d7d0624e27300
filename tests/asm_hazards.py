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
