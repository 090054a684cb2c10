"""Build-time check of the device assembly for one hazard the compiler does
not guard: the MFMAs whose accumulators live in AGPRs are written as inline
asm (``mfma32_agpr``), so the compiler neither knows they are MFMAs nor
inserts the wait states their results need before another instruction
reads or writes those registers.  The kernels end such a chain with
``mfma_agpr_wait`` (24 wait states; a 32x32 MFMA result needs 18) and keep
every other access to the accumulators after it, but the register
allocator may still place a copy of an accumulator (``v_accvgpr_read``,
``v_accvgpr_mov``) between the last MFMA and the wait, for instance at a
loop exit.  Such a copy reads a value the MFMA has not written yet, and the
result is silently wrong.

The same blindness applies in the other direction: an MFMA needs two wait
states after a VALU instruction writes one of its A or B operands, which
the compiler would insert before its own MFMAs but not before the asm.

``check_asm`` builds each kernel's control-flow graph from the assembly
text and computes, at every instruction, the fewest wait states along any
path (an ``s_nop N`` gives N + 1, any other instruction one, MFMAs none)
since an MFMA with an AGPR destination last wrote each AGPR, and since the
last VALU write of each VGPR.  It reports an instruction other than an
MFMA that names an AGPR some MFMA wrote fewer than 18 wait states before
(other AGPRs, such as those the compiler uses to hold spilled values, are
free to use), and an AGPR-destination MFMA that reads a VGPR with fewer
than 2 of the second.
"""
from __future__ import annotations

import re

WAIT_STATES = 18
OPERAND_WAIT_STATES = 2
_KERNEL = re.compile(r"^(_Z\S+):")
_LABEL = re.compile(r"^(\.L\S+):")
_AGPR = re.compile(r"\ba(\d+)\b|\ba\[(\d+):(\d+)\]")
_VREG = re.compile(r"^v\[(\d+):(\d+)\]$|^v(\d+)$")
# VALU instructions whose destination is not a VGPR, or that are not VALU
_NOT_VGPR_WRITERS = ("v_cmp", "v_cmpx", "v_readfirstlane", "v_readlane", "v_accvgpr_write",
                     "v_mfma")


def _vregs(tok: str) -> set[int]:
    m = _VREG.match(tok.strip())
    if not m:
        return set()
    if m.group(3) is not None:
        return {int(m.group(3))}
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def _kernels(text: str):
    """(name, [(lineno, instruction or label)]) per kernel."""
    name, body = None, []
    for lineno, line in enumerate(text.splitlines(), 1):
        s = line.split(";", 1)[0].strip()
        if not s:
            continue
        m = _KERNEL.match(s)
        if m:
            if name:
                yield name, body
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if _LABEL.match(s) or not s.startswith("."):
            body.append((lineno, s))
        if s.startswith(".Lfunc_end"):
            yield name, body
            name, body = None, []
    if name:
        yield name, body


def _blocks(body):
    """Split into basic blocks: (label or None, [instructions], successors)."""
    blocks, cur_label, cur = [], None, []
    for lineno, s in body:
        m = _LABEL.match(s)
        if m:
            if cur or cur_label is not None:
                blocks.append([cur_label, cur])
            cur_label, cur = m.group(1), []
            continue
        cur.append((lineno, s))
        op = s.split()[0]
        if op.startswith("s_branch") or op.startswith("s_cbranch") or op in ("s_endpgm", "s_setpc_b64"):
            blocks.append([cur_label, cur])
            cur_label, cur = None, []
    if cur or cur_label is not None:
        blocks.append([cur_label, cur])
    index = {b[0]: i for i, b in enumerate(blocks) if b[0] is not None}
    succ = []
    for i, (_, ins) in enumerate(blocks):
        out = []
        last = ins[-1][1] if ins else ""
        op = last.split()[0] if last else ""
        if op.startswith("s_branch") or op.startswith("s_cbranch"):
            target = last.split()[1]
            if target in index:
                out.append(index[target])
        if not (op.startswith("s_branch") or op in ("s_endpgm", "s_setpc_b64")) and i + 1 < len(blocks):
            out.append(i + 1)
        succ.append(out)
    return blocks, succ


def _age(ages, k, limit):
    """Advance the ages (wait states) by k, dropping those that reach limit."""
    return {r: a + k for r, a in ages.items() if a + k < limit}


def _agprs(text: str) -> set[int]:
    out = set()
    for m in _AGPR.finditer(text):
        if m.group(1) is not None:
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _run(ins, state, report):
    """state: (AGPR -> wait states since an MFMA wrote it, VGPR -> wait
    states since a VALU wrote it), both holding only the recent ones."""
    acc, recent = state
    for lineno, s in ins:
        op = s.split()[0]
        if op.startswith("v_mfma"):
            ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
            if ops[0].startswith("a"):
                for r in _vregs(ops[1]) | _vregs(ops[2]):
                    if r in recent:
                        report.append((lineno, s, f"v{r} written {recent[r]} wait states before "
                                                   f"this MFMA reads it"))
                acc = dict(acc)
                for r in _agprs(ops[0]):
                    acc[r] = 0
            continue
        if op == "s_nop":
            k = int(s.split()[1], 0) + 1
            acc = _age(acc, k, WAIT_STATES)
            recent = _age(recent, k, OPERAND_WAIT_STATES)
            continue
        if acc:
            hit = sorted(r for r in _agprs(s) if r in acc)
            if hit:
                report.append((lineno, s, f"a{hit[0]} written by an MFMA {acc[hit[0]]} wait "
                                          f"states before"))
        acc = _age(acc, 1, WAIT_STATES)
        recent = _age(recent, 1, OPERAND_WAIT_STATES)
        if op.startswith("v_") and not op.startswith(_NOT_VGPR_WRITERS):
            parts = s.split(None, 1)
            if len(parts) > 1:
                for r in _vregs(parts[1].split(",")[0]):
                    recent[r] = 0
    return acc, recent


def _merge(a, b):
    """State at a join: the fewest wait states on either path."""
    out = []
    for x, y in zip(a, b):
        m = dict(x)
        for r, age in y.items():
            m[r] = min(age, m.get(r, age))
        out.append(m)
    return tuple(out)


def check_asm(text: str) -> list[str]:
    """Violations in one assembly file, as readable strings."""
    out = []
    for name, body in _kernels(text):
        blocks, succ = _blocks(body)
        if not blocks:
            continue
        entry = [None] * len(blocks)
        entry[0] = ({}, {})
        work = [0]
        while work:
            i = work.pop()
            st = _run(blocks[i][1], entry[i], [])
            for j in succ[i]:
                new = st if entry[j] is None else _merge(entry[j], st)
                if entry[j] is None or new != entry[j]:
                    entry[j] = new
                    work.append(j)
        for i, (_, ins) in enumerate(blocks):
            if entry[i] is None:
                continue
            rep = []
            _run(ins, entry[i], rep)
            for lineno, s, why in rep:
                out.append(f"{name}: line {lineno}: '{s}': {why}")
    return out
