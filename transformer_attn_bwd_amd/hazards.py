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

``check_asm`` builds each kernel's control-flow graph from the assembly
text and computes, at every instruction, the fewest wait states since an
MFMA with an AGPR destination along any path (an ``s_nop N`` gives N + 1,
any other instruction one, MFMAs none); an instruction other than an MFMA
that names an AGPR with fewer than 18 is reported.
"""
from __future__ import annotations

import re

WAIT_STATES = 18
INF = 1 << 30
_KERNEL = re.compile(r"^(_Z\S+):")
_LABEL = re.compile(r"^(\.L\S+):")
_AGPR = re.compile(r"\ba(\d+)\b|\ba\[\d+:\d+\]")


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


def _run(ins, w, report):
    for lineno, s in ins:
        op = s.split()[0]
        if op.startswith("v_mfma"):
            if s.split(None, 1)[1].split(",")[0].strip().startswith("a"):
                w = 0
            continue
        if op == "s_nop":
            w = min(INF, w + int(s.split()[1], 0) + 1)
            continue
        if w < WAIT_STATES and _AGPR.search(s):
            report.append((lineno, s, w))
        w = min(INF, w + 1)
    return w


def check_asm(text: str) -> list[str]:
    """Violations in one assembly file, as readable strings."""
    out = []
    for name, body in _kernels(text):
        blocks, succ = _blocks(body)
        if not blocks:
            continue
        entry = [INF] * len(blocks)
        work = [0]
        seen = set()
        while work:
            i = work.pop()
            seen.add(i)
            w = _run(blocks[i][1], entry[i], [])
            for j in succ[i]:
                if w < entry[j] or j not in seen:
                    entry[j] = min(entry[j], w)
                    seen.add(j)
                    work.append(j)
        for i, (_, ins) in enumerate(blocks):
            rep = []
            _run(ins, entry[i], rep)
            for lineno, s, w in rep:
                out.append(f"{name}: line {lineno}: '{s}' {w} wait states after an "
                           f"AGPR-accumulating MFMA")
    return out
