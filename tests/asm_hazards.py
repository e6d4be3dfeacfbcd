"""Wait-state checks on gfx950 assembly for matrix products the compiler
cannot see into (inline assembly).

The hardware needs a gap, counted in wait states, between a matrix product
and a vector instruction that touches its registers.  For a product written
as inline assembly the compiler inserts none of these and takes the result as
written at issue, so it may read, copy or move the registers at once.  Two
checks cover every control-flow path of a kernel:

- dest_hazards: no instruction other than a product accumulating into
  exactly the same registers touches a product's destination before `need`
  wait states have passed (walking forward);
- source_hazards: no vector instruction writes a product's source operands
  (A, B or the accumulator) fewer than `need` wait states before it (walking
  backward).

Counting is conservative: s_nop N counts N + 1, any other instruction 1, and
both directions of every branch are followed."""
from __future__ import annotations

import re

_REG = re.compile(r"\b([av])(\d+)\b|\b([av])\[(\d+):(\d+)\]")


def regs(text):
    """(file, first, last) of every a/v register or range in text."""
    out = []
    for m in _REG.finditer(text):
        if m.group(1):
            out.append((m.group(1), int(m.group(2)), int(m.group(2))))
        else:
            out.append((m.group(3), int(m.group(4)), int(m.group(5))))
    return out


def _overlap(a, b):
    return a[0] == b[0] and a[1] <= b[2] and b[1] <= a[2]


def _operands(ins):
    parts = ins.split(None, 1)
    return [p.strip() for p in parts[1].split(",")] if len(parts) > 1 else []


def kernels(asm, pattern):
    """{symbol: [instruction or label lines]} of the kernels in the assembly
    listing whose symbol contains pattern."""
    out = {}
    for m in re.finditer(r"\n(\S+?):\s*;\s*@", asm):
        name = m.group(1)
        if pattern not in name or name.startswith("."):
            continue
        end = asm.index("s_endpgm", m.end())
        body = asm[m.end():end].split("\n")
        out[name] = [ln.split(";")[0].strip() for ln in body
                     if re.match(r"^\s+[a-z]", ln) or ln.startswith(".LBB")]
    return out


def _labels(code):
    return {ln[:-1]: i for i, ln in enumerate(code) if ln.startswith(".LBB")}


def dest_hazards(code, need_a=32, need_v=11):
    """(product, instruction, wait states) for every instruction that touches
    a product's destination too early; need_a / need_v for AGPR / VGPR
    destinations."""
    lab = _labels(code)
    hits = []
    for idx, ins in enumerate(code):
        if not ins.startswith("v_mfma"):
            continue
        ops = _operands(ins)
        dst = regs(ops[0])[0]
        need = need_a if dst[0] == "a" else need_v
        stack, seen = [(idx + 1, 0)], set()
        while stack:
            k, ws = stack.pop()
            while k < len(code) and ws < need and (k, ws) not in seen:
                seen.add((k, ws))
                o = code[k]
                if o.startswith(".LBB"):
                    k += 1
                    continue
                op = o.split()[0]
                if op == "s_nop":
                    ws += int(o.split()[1]) + 1
                    k += 1
                    continue
                if op.startswith("v_mfma"):
                    # a later product may accumulate into exactly the same
                    # registers; any other overlap is a hazard
                    oo = _operands(o)
                    d2 = regs(oo[0])
                    bad = any(_overlap(r, dst) and r != dst for r in d2)
                    for i, p in enumerate(oo[1:], 1):
                        for r in regs(p):
                            if _overlap(r, dst) and not (i == 3 and r == dst and d2 == [dst]):
                                bad = True
                    if bad:
                        hits.append((ins, o, ws))
                elif any(_overlap(r, dst) for p in _operands(o) for r in regs(p)):
                    hits.append((ins, o, ws))
                if op == "s_branch":
                    k = lab[o.split()[1]]
                    ws += 1
                    continue
                if op.startswith("s_cbranch") and o.split()[1] in lab:
                    stack.append((lab[o.split()[1]], ws + 1))
                if op in ("s_endpgm", "s_setpc_b64"):
                    break
                ws += 1
                k += 1
    return hits


def source_hazards(code, need=2):
    """(writer, product, wait states) for every vector write of a product's
    source operands fewer than need wait states before it."""
    preds = {}
    for i, o in enumerate(code):
        p = o.split()
        if p and (p[0] == "s_branch" or p[0].startswith("s_cbranch")) and len(p) > 1:
            preds.setdefault(p[1], []).append(i)
    hits = []
    for idx, ins in enumerate(code):
        if not ins.startswith("v_mfma"):
            continue
        srcs = [r for p in _operands(ins)[1:] for r in regs(p)]
        stack, seen = [(idx - 1, 0)], set()
        while stack:
            k, ws = stack.pop()
            while k >= 0 and ws < need and (k, ws) not in seen:
                seen.add((k, ws))
                o = code[k]
                if o.startswith(".LBB"):
                    for b in preds.get(o[:-1], []):   # continue before the branch, which counts 1
                        stack.append((b - 1, ws + 1))
                    if k > 0 and code[k - 1].split()[0] == "s_branch":
                        break
                    k -= 1
                    continue
                op = o.split()[0]
                if op == "s_nop":
                    ws += int(o.split()[1]) + 1
                    k -= 1
                    continue
                if op.startswith("v_") and not op.startswith("v_mfma"):
                    ops = _operands(o)
                    if ops and any(_overlap(r, s) for r in regs(ops[0]) for s in srcs):
                        hits.append((o, ins, ws))
                if op == "s_branch":
                    break
                ws += 1
                k -= 1
    return hits
