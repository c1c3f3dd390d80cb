"""Static check of MFMA result hazards in gfx950 assembly.

An MFMA writes its destination VGPRs some cycles after it issues, and gfx950 does
not interlock a later VALU or memory instruction that reads (or overwrites) those
registers: the program must leave enough wait states in between.  The compiler
inserts them within a basic block, but a read reached through a branch can be
left without them; the read then sees a stale value, and results change from run
to run.  `find_hazards` walks every control-flow path from every MFMA and reports
each non-MFMA instruction that touches one of its destination registers fewer
than `min_waits` wait states after it (`s_nop N` counts N + 1, every other
instruction 1).  MFMAs that accumulate into the same registers are exempt (the
hardware chains them); MFMAs reading them as A or B operands are reported.
"""

from __future__ import annotations

import re

_RANGE = re.compile(r"\b([va])\[(\d+):(\d+)\]")
_SINGLE = re.compile(r"\b([va])(\d+)\b")


def _regs(text: str) -> set:
    out = set()
    for m in _RANGE.finditer(text):
        out |= {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    for m in _SINGLE.finditer(text):
        out.add((m.group(1), int(m.group(2))))
    return out


def functions(asm: str) -> dict:
    """Kernel name -> body lines of each function in an assembly file."""
    funcs, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
        elif cur is not None:
            if line.startswith(".Lfunc_end"):
                cur = None
            else:
                funcs[cur].append(line)
    return funcs


def _blocks(body):
    blocks, label, ins = [], "entry", []
    for line in body:
        m = re.match(r"^\.L(BB\d+_\d+):", line) or re.match(r"^; %bb\.(\d+):", line)
        if m:
            blocks.append((label, ins))
            label, ins = m.group(1), []
            continue
        t = line.strip()
        if not t or t.startswith((";", ".")):
            continue
        ins.append(t.split(";")[0].strip())
    blocks.append((label, ins))
    index = {lab: i for i, (lab, _) in enumerate(blocks)}
    succ = []
    for i, (_, ins) in enumerate(blocks):
        last = ins[-1] if ins else ""
        op = last.split()[0] if last else ""
        s = []
        if op.startswith("s_cbranch") or op == "s_branch":
            tgt = last.split()[-1]
            tgt = tgt[2:] if tgt.startswith(".L") else tgt
            if tgt in index:
                s.append(index[tgt])
        if op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    return blocks, succ


def find_hazards(body, min_waits: int = 8):
    """(mfma, reader, wait states) for every too-close use of an MFMA result."""
    blocks, succ = _blocks(body)
    found = {}
    for bi, (_, ins) in enumerate(blocks):
        for ii, mf in enumerate(ins):
            op = mf.split()[0]
            if not op.startswith("v_mfma"):
                continue
            dst = _regs(mf[len(op):].split(",")[0])
            stack, seen = [(bi, ii + 1, 0)], set()
            while stack:
                b, i, w = stack.pop()
                if w >= min_waits or (b, i, w) in seen:
                    continue
                seen.add((b, i, w))
                code = blocks[b][1]
                if i >= len(code):
                    stack.extend((s, 0, w) for s in succ[b])
                    continue
                u = code[i]
                uop = u.split()[0]
                operands = u[len(uop):]
                if uop.startswith("v_mfma"):
                    parts = operands.split(",")
                    if not _regs(",".join(parts[1:3])).isdisjoint(dst):
                        found.setdefault((mf, u), w)
                        continue
                    if _regs(parts[0]) >= dst:
                        continue  # accumulates into the same registers
                elif uop == "s_nop":
                    stack.append((b, i + 1, w + int(u.split()[1], 0) + 1))
                    continue
                elif uop.startswith(("v_", "global_", "buffer_", "ds_", "scratch_", "flat_")):
                    if not _regs(operands).isdisjoint(dst):
                        found[(mf, u)] = min(w, found.get((mf, u), w))
                        continue
                stack.append((b, i + 1, w + 1))
    return [(mf, u, w) for (mf, u), w in found.items()]
