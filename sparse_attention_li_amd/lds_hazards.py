"""Build-time check of the kernels' explicitly awaited LDS reads.

Some kernels issue LDS reads as instructions of their own (inline assembly)
and wait for them with explicit lgkmcnt waits placed later, so that the reads
overlap with matrix instructions.  The compiler does not know that such a
register is still being written until the wait: if it spilled, copied or
otherwise read that register in between, the value would be read early.

This module scans the compiled gfx950 assembly of the named kernels and
reports every instruction that reads or overwrites a vector register whose
LDS load may still be in flight.  It models the LDS counter per path: DS
operations complete in order, so lgkmcnt(N) leaves at most the N most recent
DS operations in flight, whatever scalar loads share the counter.  The
function is split into basic blocks (labels and branches); the in-flight
queue entering a block is the merge of its predecessors' queues -- aligned
from the most recent operation, each position the union of the registers any
path may still be loading there -- iterated to a fixed point, so reads issued
at the end of a loop body are checked at the loop head and a wait on a branch
that may be skipped clears nothing after the join.
"""
from __future__ import annotations

import re

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")
_DS_NO_RESULT = re.compile(r"^ds_(write|store|add_u32|add_u64|sub_u32|min_|max_|and_b|or_b|xor_b|inc_u|dec_u|nop|gws|append|consume)")
_MAX_QUEUE = 32  # older in-flight operations are folded into one entry (conservative)


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


def _cap(q: tuple) -> tuple:
    if len(q) <= _MAX_QUEUE:
        return q
    head = frozenset().union(*q[: len(q) - _MAX_QUEUE + 1])
    return (head,) + q[len(q) - _MAX_QUEUE + 1:]


def _merge(a: tuple, b: tuple) -> tuple:
    """Queues (oldest first) of two paths, aligned at their most recent entries."""
    n = max(len(a), len(b))
    pa = (frozenset(),) * (n - len(a)) + a
    pb = (frozenset(),) * (n - len(b)) + b
    return tuple(x | y for x, y in zip(pa, pb))


def _step(raw: str, q: tuple, hazards: list | None) -> tuple:
    """One instruction: returns the new queue, appending hazards if asked."""
    line = raw.split(";")[0].strip()
    op, _, rest = line.partition(" ")
    if op == "s_waitcnt":
        m = re.search(r"lgkmcnt\((\d+)\)", rest)
        if m:
            n = int(m.group(1))
            q = q[len(q) - n:] if n < len(q) else q
            if n == 0:
                q = ()
        return q
    ops = _split_operands(rest)
    busy = frozenset().union(*q) if q else frozenset()
    if op.startswith("ds_"):
        returns = not _DS_NO_RESULT.match(op) or "_rtn" in op
        dst = _regs(ops[0]) if (returns and ops) else set()
        srcs = set().union(*[_regs(o) for o in (ops[1:] if returns else ops)]) if ops else set()
        if hazards is not None:
            for r in sorted((srcs | dst) & busy):
                hazards.append((raw.strip(), r))
        return _cap(q + (frozenset(dst),))
    is_store = "store" in op or op.startswith("buffer_wbl2")
    dst = set() if is_store or not ops else _regs(ops[0])
    srcs = set().union(*[_regs(o) for o in (ops if is_store else ops[1:])]) if ops else set()
    if hazards is not None:
        for r in sorted((srcs | dst) & busy):
            hazards.append((raw.strip(), r))
    return q


def _blocks(lines: list):
    """Basic blocks: (label, instruction lines, successor labels / None for
    the fall-through block, ends the function)."""
    blocks, label, insts = [], None, []

    def close(term):
        nonlocal label, insts
        blocks.append([label, insts, term])
        label, insts = None, []

    for raw in lines:
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":"):
            if insts or label is not None:
                close(None)
            label = line[:-1]
            continue
        if line.startswith("."):
            continue
        insts.append(raw)
        op, _, rest = line.partition(" ")
        if op == "s_endpgm" or op.startswith("s_setpc") or op == "s_branch" or op.startswith("s_cbranch"):
            close(line)
    if insts or label is not None:
        close(None)
    index = {b[0]: i for i, b in enumerate(blocks) if b[0] is not None}
    succ = []
    for i, (_, _, term) in enumerate(blocks):
        nxt = [i + 1] if i + 1 < len(blocks) else []
        if term is None:
            succ.append(nxt)
            continue
        op, _, rest = term.partition(" ")
        tgt = rest.split(",")[0].strip()
        if op == "s_endpgm" or op.startswith("s_setpc"):
            succ.append([])
        elif op == "s_branch":
            succ.append([index[tgt]] if tgt in index else [])
        else:
            succ.append(([index[tgt]] if tgt in index else []) + nxt)
    return [(b[1]) for b in blocks], succ


def scan_function(lines: list) -> list:
    """Returns (line text, register) for every hazard in one function body."""
    insts, succ = _blocks(lines)
    if not insts:
        return []
    n = len(insts)
    state_in = [None] * n
    state_in[0] = ()
    work = [0]
    while work:
        i = work.pop()
        q = state_in[i]
        for raw in insts[i]:
            q = _step(raw, q, None)
        for j in succ[i]:
            new = q if state_in[j] is None else _merge(state_in[j], q)
            if new != state_in[j]:
                state_in[j] = new
                work.append(j)
    hazards, seen = [], set()
    for i in range(n):
        if state_in[i] is None:
            continue  # unreachable
        q, found = state_in[i], []
        for raw in insts[i]:
            q = _step(raw, q, found)
        for h in found:
            if h not in seen:
                seen.add(h)
                hazards.append(h)
    return hazards


def check_asm(asm: str, kernels: tuple) -> list:
    """Scans every function whose name contains one of `kernels`, from its
    label to its end marker."""
    found = []
    lines = asm.splitlines()
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\S+):", lines[i])
        if m and any(k in m.group(1) for k in kernels):
            name, body = m.group(1), []
            i += 1
            while i < len(lines) and not lines[i].startswith(".Lfunc_end"):
                body.append(lines[i])
                i += 1
            for text, reg in scan_function(body):
                found.append((name, text, "%s%d" % reg))
        i += 1
    return found
