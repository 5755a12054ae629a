"""Build-time check of the gfx950 assembly of libdbd's kernels.

The kernels issue their direct-to-LDS loads (global_load_lds_dwordx4) from
inline assembly, so the compiler's hazard recognizer does not see their
operands.  A VMEM instruction that reads an SGPR needs five wait states after
a VALU instruction wrote that SGPR (v_readlane_b32 reloading a spilled SGPR
is the usual writer), and an LDS DMA needs them after a VALU write of M0;
with fewer, the load can use a stale base address.  The check walks back
from every such load over every path that reaches it (the fall-through path
and, at a block label, every branch to it) and reports a VALU write of its
SGPR base pair or of M0 inside the last five wait states (s_nop N counts
N + 1).  build.py runs it
on the assembly that hipcc -save-temps keeps, so the code checked is the
code linked.
"""
from __future__ import annotations

import re

WAIT_STATES = 5
_DMA = re.compile(r"^global_load_lds_dword\w*\s+(?P<v>v\S+),\s+(?P<base>s\[(\d+):(\d+)\]|off)")
_KERNEL = re.compile(r"^(_Z\w+|[A-Za-z_]\w*):")
_SGPR = re.compile(r"^s\[?(\d+)(?::(\d+))?\]?$")


def _instr(line: str) -> str | None:
    t = line.split(";", 1)[0].strip()
    if not t or t.startswith(".") or t.endswith(":"):
        return None
    return t


_BRANCH = re.compile(r"^s_(?:branch|cbranch_\w+)\s+(\S+)")
_NO_FALL_THROUGH = ("s_branch", "s_setpc_b64", "s_endpgm")


def _writes(p: str, regs: set[int]) -> bool:
    """True if instruction p is a VALU instruction writing M0 or an SGPR in
    regs."""
    op = p.split()[0]
    if not op.startswith("v_") or len(p.split()) < 2:
        return False
    dst = p.split()[1].rstrip(",")
    if dst == "m0":
        return True
    s = _SGPR.match(dst)
    if not s:
        return False
    lo = int(s.group(1))
    hi = int(s.group(2) or lo)
    return bool(regs & set(range(lo, hi + 1)))


def scan(asm_text: str) -> tuple[int, list[tuple[str, int, str, str]]]:
    """Returns (number of LDS DMA instructions, hazards as (kernel, line,
    DMA instruction, offending writer)).  From each DMA the walk goes back
    over every path that reaches it within five wait states: the
    fall-through path and, at a block label, every branch to that label."""
    lines = asm_text.splitlines()
    branches: dict[str, list[int]] = {}
    for i, raw in enumerate(lines):
        t = _instr(raw)
        b = _BRANCH.match(t) if t else None
        if b:
            branches.setdefault(b.group(1), []).append(i)

    def walk(j: int, ws: int, regs: set[int], seen: set[tuple[int, int]]) -> str | None:
        # j: the line before the instruction reached so far, ws: wait states so far
        while j >= 0 and ws < WAIT_STATES:
            if (j, ws) in seen:
                return None
            seen.add((j, ws))
            raw = lines[j]
            st = raw.strip()
            if st.endswith(":") and not st.startswith(";"):
                if not st.startswith("."):
                    return None                         # the kernel's entry
                label = st[:-1]
                for b in branches.get(label, []):       # paths that jump here
                    # the branch instruction itself is one wait state
                    h = walk(b - 1, ws + 1, regs, seen)
                    if h:
                        return h
                # fall-through: only if the previous instruction can fall through
                k = j - 1
                while k >= 0 and _instr(lines[k]) is None and not (
                        lines[k].strip().endswith(":") and not lines[k].strip().startswith(";")):
                    k -= 1
                if k >= 0 and _instr(lines[k]) and _instr(lines[k]).split()[0] in _NO_FALL_THROUGH:
                    return None
                j -= 1
                continue
            p = _instr(raw)
            j -= 1
            if p is None:
                continue
            op = p.split()[0]
            if op == "s_nop":
                ws += int(p.split()[1].rstrip(","), 0) + 1
                continue
            if _writes(p, regs):
                return p
            ws += 1
        return None

    kernel = "?"
    n = 0
    hazards = []
    for i, raw in enumerate(lines):
        m = _KERNEL.match(raw)
        if m and not raw.startswith("."):
            kernel = m.group(1)
        t = _instr(raw)
        if t is None:
            continue
        d = _DMA.match(t)
        if not d:
            continue
        n += 1
        regs = set()
        if d.group("base") != "off":
            regs = {int(d.group(3)), int(d.group(4))}
        h = walk(i - 1, 0, regs, set())
        if h:
            hazards.append((kernel, i + 1, t, h))
    return n, hazards
