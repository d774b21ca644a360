"""Build-time check of the hand-placed MFMAs in the generated gfx950 assembly.

The bf16 prefill kernel issues its MFMAs through inline asm (to choose their
register files).  The compiler's hazard recognizer does not look inside asm
statements, so it does not insert the wait states that CDNA3/CDNA4 require
around them.  This module scans the assembly for every MFMA inside an asm
block and checks, along every control-flow path,
  * before it: no vector ALU instruction writes one of its source registers
    within the two preceding wait states;
  * after it: no vector ALU instruction other than an MFMA reads or writes
    its destination within the following 19 wait states (more than a 32x32
    MFMA's result latency);
where ``s_nop N`` counts N + 1 wait states and any other instruction 1.
Paths are followed through branches (both ways of a conditional branch) and,
backwards, into every branch that jumps to a label.
"""
from __future__ import annotations

import re
import sys

_RANGE = re.compile(r"([va])\[(\d+):(\d+)\]")
_SINGLE = re.compile(r"([va])(\d+)$")
_LABEL = re.compile(r"^([\w.$]+):")


def _regs(tok: str) -> set:
    tok = tok.strip()
    m = _RANGE.match(tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _SINGLE.match(tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


class _Code:
    def __init__(self, asm: str):
        self.items = []          # (kind, text, in_asm): kind 'i' instruction or 'L' label
        in_asm = False
        for raw in asm.split("\n"):
            s = raw.strip()
            if not s:
                continue
            if s.startswith(";;#ASMSTART"):
                in_asm = True
            elif s.startswith(";;#ASMEND"):
                in_asm = False
            elif s.startswith(";") or (s.startswith(".") and not _LABEL.match(s)):
                continue
            elif _LABEL.match(s):
                self.items.append(("L", _LABEL.match(s).group(1), in_asm))
            else:
                self.items.append(("i", s.split(";")[0].strip(), in_asm))
        self.label_at = {t: i for i, (k, t, _) in enumerate(self.items) if k == "L"}
        self.jumps_to = {}
        for i, (k, t, _) in enumerate(self.items):
            if k == "i" and (t.startswith("s_cbranch") or t.startswith("s_branch")):
                target = t.split()[-1]
                self.jumps_to.setdefault(target, []).append(i)

    @staticmethod
    def op(text: str) -> str:
        return text.split()[0]

    @staticmethod
    def operands(text: str) -> list:
        return [o.strip() for o in text.split(None, 1)[1].split(",")] if " " in text else []

    def asm_mfmas(self):
        for i, (k, t, a) in enumerate(self.items):
            if k == "i" and a and t.startswith("v_mfma"):
                yield i, t


def _cost(text: str) -> int:
    op = text.split()[0]
    return int(text.split()[1], 0) + 1 if op == "s_nop" else 1


def _is_valu(text: str) -> bool:
    op = text.split()[0]
    return op.startswith("v_") and not op.startswith("v_mfma")


def _scan_back(code: _Code, idx: int, budget: int, srcs: set, seen: set, out: list, mfma: str):
    """Instructions before position idx (exclusive) within budget wait states."""
    j = idx - 1
    while budget > 0 and j >= 0:
        kind, text, _ = code.items[j]
        if kind == "L":
            for b in code.jumps_to.get(text, []):
                key = (b, budget)
                if key not in seen:
                    seen.add(key)
                    # the branch itself is one instruction on that path
                    _scan_back(code, b + 1, budget, srcs, seen, out, mfma)
            # fall-through predecessor exists unless the previous instruction ends the path
            k = j - 1
            while k >= 0 and code.items[k][0] == "L":
                k -= 1
            if k >= 0 and code.items[k][0] == "i" and code.op(code.items[k][1]) in ("s_branch", "s_endpgm"):
                return
            j -= 1
            continue
        if _is_valu(text) and _regs(code.operands(text)[0] if code.operands(text) else "") & srcs:
            out.append(f"{text}  ->  {mfma}")
        budget -= _cost(text)
        j -= 1


def _scan_fwd(code: _Code, idx: int, budget: int, dst: set, seen: set, out: list, mfma: str):
    """Instructions after position idx (exclusive) within budget wait states."""
    j = idx + 1
    while budget > 0 and j < len(code.items):
        kind, text, _ = code.items[j]
        if kind == "L":
            j += 1
            continue
        op = code.op(text)
        if _is_valu(text):
            regs = set().union(*[_regs(o) for o in code.operands(text)]) if code.operands(text) else set()
            if regs & dst:
                out.append(f"{mfma}  ->  {text}")
        budget -= _cost(text)
        if op == "s_endpgm":
            return
        if op.startswith("s_cbranch") or op == "s_branch":
            target = code.label_at.get(text.split()[-1])
            if target is not None and (target, budget) not in seen:
                seen.add((target, budget))
                _scan_fwd(code, target, budget, dst, seen, out, mfma)
            if op == "s_branch":
                return
        j += 1


def check(asm: str, wait_states: int = 2) -> list:
    """Vector writes to an asm MFMA's source registers too soon before it."""
    code = _Code(asm)
    out = []
    for idx, text in code.asm_mfmas():
        srcs = set().union(*[_regs(o) for o in code.operands(text)[1:4]])
        _scan_back(code, idx, wait_states, srcs, set(), out, text)
    return out


def check_results(asm: str, wait_states: int = 19) -> list:
    """Vector instructions touching an asm MFMA's destination too soon after it."""
    code = _Code(asm)
    out = []
    for idx, text in code.asm_mfmas():
        dst = _regs(code.operands(text)[0])
        _scan_fwd(code, idx, wait_states, dst, set(), out, text)
    return out


def check_all(asm: str) -> list:
    return check(asm) + check_results(asm)


def count_asm_mfma(asm: str) -> int:
    return sum(1 for _ in _Code(asm).asm_mfmas())


if __name__ == "__main__":
    text = open(sys.argv[1]).read()
    found = check_all(text)
    for p in found:
        print(p)
    print(f"{count_asm_mfma(text)} asm MFMAs, {len(found)} problems")
    sys.exit(1 if found else 0)
