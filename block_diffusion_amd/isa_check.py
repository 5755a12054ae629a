"""Build-time check of the gfx950 assembly of libdbd's kernels.

The kernels issue their direct-to-LDS loads (global_load_lds_dwordx4) from
inline assembly, so the compiler's hazard recognizer does not see their
operands.  A VMEM instruction that reads an SGPR needs five wait states after
a VALU instruction wrote that SGPR (v_readlane_b32 reloading a spilled SGPR
is the usual writer), and an LDS DMA needs them after a VALU write of M0;
with fewer, the load can use a stale base address.  The check walks back
from every such load along the fall-through path (across block labels,
stopping where the previous instruction is an unconditional branch; other
branch sources are not followed) and reports a VALU write of its SGPR base
pair or of M0 inside the last five wait states (s_nop N counts N + 1).  The
kernels' DMA assembly starts with s_nop 4, so every path is covered; the
check guards that property in the code actually built.  build.py runs it
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


def scan(asm_text: str) -> tuple[int, list[tuple[str, int, str, str]]]:
    """Returns (number of LDS DMA instructions, hazards as (kernel, line,
    DMA instruction, offending writer))."""
    lines = asm_text.splitlines()
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
        ws = 0
        j = i - 1
        crossed = False
        while j >= 0 and ws < WAIT_STATES:
            prev = lines[j]
            j -= 1
            st = prev.strip()
            if st.endswith(":") and not st.startswith(";"):
                if _KERNEL.match(st) and not st.startswith("."):
                    break                               # the kernel's entry
                crossed = True                          # a block label: follow the fall-through
                continue
            p = _instr(prev)
            if p is None:
                continue
            op = p.split()[0]
            if crossed and op in ("s_branch", "s_setpc_b64", "s_endpgm"):
                break                                   # no fall-through into the block
            crossed = False
            if op == "s_nop":
                ws += int(p.split()[1].rstrip(","), 0) + 1
                continue
            if op.startswith("v_"):
                dst = p.split()[1].rstrip(",") if len(p.split()) > 1 else ""
                if dst == "m0":
                    hazards.append((kernel, i + 1, t, p))
                    break
                s = _SGPR.match(dst)
                if s:
                    lo = int(s.group(1))
                    hi = int(s.group(2) or lo)
                    if regs & set(range(lo, hi + 1)):
                        hazards.append((kernel, i + 1, t, p))
                        break
            ws += 1
    return n, hazards
