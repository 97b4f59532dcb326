"""Dependency hazards around hand-written matrix-core instructions in gfx950 ISA.

CDNA's matrix cores do not interlock every register dependency: software
must leave a number of independent instructions or wait states between, for
example, a vector ALU write of a register and a matrix op that reads it, or
a matrix op's result and a vector instruction that reads it.  The compiler
inserts these for the matrix ops it emits itself, but an inline-asm matrix op
is opaque to it: any move it schedules right before or after one is a silent
read of stale data.

This module scans the assembly of our own build (``hipcc -S``) over its
control-flow graph (pending hazards flow along every branch, including loop
back edges) and reports, for each place where an inline-asm matrix op is
involved:

  A  a VALU write of a v/a register, then a matrix op reading it (any source)
     within VALU_TO_MFMA wait states;
  B  a matrix op's result, then any non-matrix instruction touching it
     within MFMA_RESULT wait states;
  C  a matrix op's result, then a matrix op reading it as source A or B
     within MFMA_RESULT wait states;
  D  an EXEC write, then a matrix op within EXEC_TO_MFMA wait states.

MFMA_RESULT is deliberately above what the 8-pass 32x32x16 bf16 op needs.
"""

from __future__ import annotations

import re
from dataclasses import dataclass

VALU_TO_MFMA = 2
MFMA_RESULT = 19
EXEC_TO_MFMA = 4

_REG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")
_BRANCH_ENDS = ("s_branch", "s_cbranch", "s_endpgm", "s_setpc_b64")


@dataclass(frozen=True)
class Inst:
    line: int
    op: str
    args: tuple
    asm: bool  # written by hand (inside an inline-asm block)


@dataclass(frozen=True)
class Hazard:
    kind: str
    line: int       # the instruction that reads or touches too early
    source: int     # the instruction that made the hazard
    missing: int    # wait states short

    def __str__(self):
        return f"{self.kind}: line {self.line} <- line {self.source}: {self.missing} wait state(s) missing"


def regs(text: str) -> frozenset:
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            for r in range(int(m.group(4)), int(m.group(5)) + 1):
                out.add((m.group(3), r))
    return frozenset(out)


def parse(asm_text: str):
    """Basic blocks of every function in the file: list of (label, insts, succ)."""
    blocks = [[None, []]]
    in_asm = False
    for no, raw in enumerate(asm_text.split("\n"), 1):
        stripped = raw.strip()
        if stripped.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if stripped.startswith(";;#ASMEND"):
            in_asm = False
            continue
        lab = re.match(r"^(\.LBB\d+_\d+):", raw)
        if lab or raw.startswith("; %bb.") or re.match(r"^[A-Za-z_][\w.$]*:\s*(;.*)?$", raw):
            blocks.append([lab.group(1) if lab else None, []])
            continue
        code = raw.split(";")[0].strip()
        if not code or code.startswith("."):
            continue
        op = code.split()[0]
        rest = code[len(op):]
        args = tuple(a.strip() for a in rest.split(",")) if rest.strip() else ()
        blocks[-1][1].append(Inst(no, op, args, in_asm))
        if op.startswith(_BRANCH_ENDS):
            blocks.append([None, []])
    blocks = [b for b in blocks if b[0] or b[1]]
    index = {b[0]: i for i, b in enumerate(blocks) if b[0]}
    out = []
    for i, (label, insts) in enumerate(blocks):
        last = insts[-1] if insts else None
        succ = []
        if last is not None and last.op == "s_branch":
            succ.append(index[last.args[0]])
        elif last is not None and last.op.startswith("s_cbranch"):
            succ.append(index[last.args[0]])
            if i + 1 < len(blocks):
                succ.append(i + 1)
        elif last is not None and last.op in ("s_endpgm", "s_setpc_b64"):
            pass
        elif i + 1 < len(blocks):
            succ.append(i + 1)
        out.append((label, insts, succ))
    return out


def _age(state, n):
    return frozenset((k, w - n, d, src, a) for (k, w, d, src, a) in state if w - n > 0)


def _step(state, inst: Inst, report):
    if inst.op == "s_nop":
        return _age(state, int(inst.args[0], 0) + 1)
    if inst.op.startswith("v_mfma"):
        dst = regs(inst.args[0])
        src = regs(",".join(inst.args[1:4]))
        src_ab = regs(",".join(inst.args[1:3]))
        for (k, w, d, s, a) in state:
            if k == "V" and d & src and inst.asm:
                report("A", inst.line, s, w)
            elif k == "M" and d & src_ab and (a or inst.asm):
                report("C", inst.line, s, w)
            elif k == "E" and inst.asm:
                report("D", inst.line, s, w)
        nxt = set(_age(state, 1))
        nxt.add(("M", MFMA_RESULT, dst, inst.line, inst.asm))
        return frozenset(nxt)
    touched = regs(",".join(inst.args))
    for (k, w, d, s, a) in state:
        if k == "M" and d & touched and (a or inst.asm):
            report("B", inst.line, s, w)
    nxt = set(_age(state, 1))
    if (inst.op.startswith("v_") and inst.args and not inst.op.startswith("v_cmp")
            and not inst.op.startswith("v_read")):
        d = regs(inst.args[0])
        if d:
            nxt.add(("V", VALU_TO_MFMA, d, inst.line, inst.asm))
    if (inst.args and inst.args[0].startswith("exec")) or inst.op.startswith("v_cmpx"):
        nxt.add(("E", EXEC_TO_MFMA, frozenset(), inst.line, inst.asm))
    return frozenset(nxt)


def check(asm_text: str) -> list:
    """All hazards in the file, sorted by line."""
    blocks = parse(asm_text)
    entry = [frozenset() for _ in blocks]
    done = [None] * len(blocks)
    found = {}

    def report(kind, line, source, missing):
        key = (kind, line, source)
        found[key] = max(found.get(key, 0), missing)

    work = list(range(len(blocks)))[::-1]
    while work:
        i = work.pop()
        state = entry[i]
        if done[i] == state:
            continue
        done[i] = state
        for inst in blocks[i][1]:
            state = _step(state, inst, report)
        for s in blocks[i][2]:
            merged = entry[s] | state
            if merged != entry[s] or done[s] is None:
                entry[s] = merged
                work.append(s)
    return [Hazard(k, l, s, m) for (k, l, s), m in sorted(found.items(), key=lambda kv: kv[0][1])]
