"""Build-time check of the hand-placed MFMAs in the generated gfx950 assembly.

The bf16 prefill kernel issues its output-accumulator MFMAs through inline asm
(to keep the accumulators in AGPRs).  The compiler's hazard recognizer does
not look inside asm statements, so it does not insert the two wait states
that CDNA3/CDNA4 require between a vector ALU instruction writing a VGPR and
an MFMA reading that VGPR as a source operand.  This module scans the
assembly for every MFMA inside an asm block and checks that no vector ALU
instruction writes any of its source registers within the two preceding wait
states (``s_nop N`` counts N + 1, any other instruction 1).  A label inside
that window is reported as well: the predecessor on another path is unknown.
"""
from __future__ import annotations

import re
import sys

_RANGE = re.compile(r"([va])\[(\d+):(\d+)\]")
_SINGLE = re.compile(r"([va])(\d+)$")


def _regs(tok: str) -> set:
    tok = tok.strip()
    m = _RANGE.match(tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _SINGLE.match(tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _lines(asm: str):
    """(kind, text): 'i' instruction, 'L' label, 'A' asm start, 'E' asm end."""
    out = []
    for raw in asm.split("\n"):
        s = raw.strip()
        if not s:
            continue
        if s.startswith(";;#ASMSTART"):
            out.append(("A", s))
        elif s.startswith(";;#ASMEND"):
            out.append(("E", s))
        elif s.startswith(";") or (s.startswith(".") and not s.startswith(".LBB")):
            continue
        elif re.match(r"^[\w.$]+:", s):
            out.append(("L", s))
        else:
            out.append(("i", s.split(";")[0].strip()))
    return out


def check(asm: str, wait_states: int = 2) -> list:
    """Problems found (empty when every asm MFMA is preceded by enough wait states)."""
    items = _lines(asm)
    problems = []
    in_asm = False
    for idx, (kind, txt) in enumerate(items):
        if kind == "A":
            in_asm = True
            continue
        if kind == "E":
            in_asm = False
            continue
        if kind != "i" or not in_asm or not txt.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in txt.split(None, 1)[1].split(",")]
        srcs = set().union(*[_regs(o) for o in ops[1:4]])
        ws, j = 0, idx - 1
        while ws < wait_states and j >= 0:
            k2, t2 = items[j]
            if k2 == "L":
                problems.append(f"label within {wait_states} wait states of: {txt}")
                break
            if k2 == "i":
                op = t2.split()[0]
                if op == "s_nop":
                    ws += int(t2.split()[1], 0) + 1
                    j -= 1
                    continue
                if op.startswith("v_") and not op.startswith("v_mfma"):
                    dst = _regs(t2.split(None, 1)[1].split(",")[0]) if " " in t2 else set()
                    if dst & srcs:
                        problems.append(f"{t2}  ->  {txt}")
                ws += 1
            j -= 1
    return problems


def count_asm_mfma(asm: str) -> int:
    n, in_asm = 0, False
    for kind, txt in _lines(asm):
        if kind == "A":
            in_asm = True
        elif kind == "E":
            in_asm = False
        elif kind == "i" and in_asm and txt.startswith("v_mfma"):
            n += 1
    return n


if __name__ == "__main__":
    text = open(sys.argv[1]).read()
    found = check(text)
    for p in found:
        print(p)
    print(f"{count_asm_mfma(text)} asm MFMAs, {len(found)} problems")
    sys.exit(1 if found else 0)
