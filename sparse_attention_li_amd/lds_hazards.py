"""Build-time check of the attention kernels' explicitly awaited LDS reads.

Some kernels issue LDS reads as instructions of their own (inline assembly)
and wait for them with explicit lgkmcnt waits placed later, so that the reads
overlap with matrix instructions.  The compiler does not know that such a
register is still being written until the wait: if it spilled, copied or
otherwise read that register in between, the value would be read early.

This module scans the compiled gfx950 assembly of the named kernels in
program order, models the LDS counter (DS operations complete in order, so
lgkmcnt(N) leaves at most the N most recent DS operations in flight, whatever
scalar loads share the counter), and reports every instruction that reads or
overwrites a vector register whose LDS load may still be in flight.  The scan is linear: at a backward branch the pending
set is carried into the code that follows, which can only add reports.
"""
from __future__ import annotations

import re

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")
_DS_NO_RESULT = re.compile(r"^ds_(write|store|add_u32|add_u64|sub_u32|min_|max_|and_b|or_b|xor_b|inc_u|dec_u|nop|gws|append|consume)")


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            for r in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add((kind, r))
    return out


def _split_operands(rest: str) -> list:
    ops, depth, cur = [], 0, ""
    for ch in rest:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            ops.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        ops.append(cur.strip())
    return ops


def scan_function(lines: list) -> list:
    """Returns (line text, register) for every hazard in one function body."""
    pending = []  # FIFO of register sets, one per outstanding DS operation
    hazards = []
    for raw in lines:
        line = raw.split(";")[0].strip()
        if not line or line.endswith(":") or line.startswith("."):
            continue
        op, _, rest = line.partition(" ")
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", rest)
            if m:
                n = int(m.group(1))
                pending = pending[len(pending) - n:] if n < len(pending) else pending
            continue
        ops = _split_operands(rest)
        busy = set().union(*pending) if pending else set()
        if op.startswith("ds_"):
            returns = not _DS_NO_RESULT.match(op) or "_rtn" in op
            dst = _regs(ops[0]) if (returns and ops) else set()
            srcs = set().union(*[_regs(o) for o in (ops[1:] if returns else ops)]) if ops else set()
            for r in sorted((srcs | dst) & busy):
                hazards.append((raw.strip(), r))
            pending.append(dst)
            continue
        is_store = "store" in op or op.startswith("buffer_wbl2")
        dst = set() if is_store or not ops else _regs(ops[0])
        srcs = set().union(*[_regs(o) for o in (ops if is_store else ops[1:])]) if ops else set()
        for r in sorted((srcs | dst) & busy):
            hazards.append((raw.strip(), r))
    return hazards


def check_asm(asm: str, kernels: tuple) -> list:
    """Scans every function whose name contains one of `kernels`."""
    found = []
    lines = asm.splitlines()
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\S+):", lines[i])
        if m and any(k in m.group(1) for k in kernels):
            name, body = m.group(1), []
            i += 1
            while i < len(lines) and not lines[i].strip().startswith("s_endpgm"):
                body.append(lines[i])
                i += 1
            for text, reg in scan_function(body):
                found.append((name, text, "%s%d" % reg))
        i += 1
    return found
