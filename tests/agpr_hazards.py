"""Static check of the wait states around the kernels' asm MFMAs (host-side test helper).

The many-row decode kernel writes its P.V MFMAs as asm with the output accumulators in
AGPRs; the compiler's hazard recognizer does not look inside asm, so the kernel inserts
the required wait states itself.  This module checks the compiled assembly for both
directions:

  * an MFMA writing AGPRs, then any non-MFMA instruction reading one of those AGPRs (a
    copy the compiler placed at a join, an accvgpr read, a store): at least
    MFMA_TO_READ wait states on every path (a 16-pass MFMA needs at most 20), found by
    propagating each AGPR's minimum distance over the control-flow graph of basic
    blocks;
  * a VALU write of a VGPR, then an asm MFMA reading it: at least VALU_TO_ASM_MFMA
    instructions in between within the block.

Each instruction counts one wait state and `s_nop N` counts N + 1.
"""
from __future__ import annotations

import re

MFMA_TO_READ = 20
VALU_TO_ASM_MFMA = 3


def _blocks(lines):
    """Basic blocks of one function: (label, [(asm_flag, instruction)])."""
    blocks, cur, in_asm = [], ["entry", []], False
    for raw in lines:
        l = raw.strip()
        if l.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if l.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if re.match(r"^\.LBB\d+_\d+:", raw):
            blocks.append(cur)
            cur = [raw.split(":")[0], []]
            continue
        if not raw.startswith("\t") or l.startswith(";") or l.startswith("."):
            continue
        cur[1].append((in_asm, l))
        op = l.split()[0]
        if op.startswith("s_cbranch") or op in ("s_branch", "s_endpgm") or op.startswith("s_setpc"):
            blocks.append(cur)
            cur = [None, []]
    blocks.append(cur)
    return [b for b in blocks if b[1] or b[0]]


def _successors(blocks):
    idx = {b[0]: n for n, b in enumerate(blocks) if b[0]}
    out = []
    for n, (_, ins) in enumerate(blocks):
        last = ins[-1][1] if ins else ""
        op = last.split()[0] if last else ""
        if op.startswith("s_cbranch"):
            out.append([idx[last.split()[1]]] + ([n + 1] if n + 1 < len(blocks) else []))
        elif op == "s_branch":
            out.append([idx[last.split()[1]]])
        elif op == "s_endpgm" or op.startswith("s_setpc"):
            out.append([])
        else:
            out.append([n + 1] if n + 1 < len(blocks) else [])
    return out


def _agprs(tok):
    """AGPR numbers named by one operand token (a7, a[4:7])."""
    m = re.match(r"a\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"a(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _regs(tok):
    """VGPR numbers named by one operand token (v7, v[4:7])."""
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operands(l):
    args = l.split(None, 1)[1] if " " in l else ""
    return [t.strip() for t in re.split(r",(?![^\[]*\])", args)]


def _cost(l):
    op = l.split()[0]
    return int(l.split()[1], 0) + 1 if op == "s_nop" else 1


def _step(state, l):
    """Wait states since the last MFMA write, per AGPR (entries at MFMA_TO_READ dropped)."""
    c = _cost(l)
    out = {r: w + c for r, w in state.items() if w + c < MFMA_TO_READ}
    op = l.split()[0]
    if op.startswith("v_mfma"):
        for r in _agprs(_operands(l)[0]):
            out[r] = 0
    return out


def _join(a, b):
    out = dict(a)
    for r, w in b.items():
        out[r] = min(w, out.get(r, w))
    return out


def check_function(lines):
    """Violations in one function's assembly lines: list of strings."""
    blocks = _blocks(lines)
    succ = _successors(blocks)
    entry = [None] * len(blocks)
    entry[0] = {}
    changed = True
    while changed:
        changed = False
        for n, (_, ins) in enumerate(blocks):
            if entry[n] is None:
                continue
            st = entry[n]
            for _, l in ins:
                st = _step(st, l)
            for m in succ[n]:
                new = st if entry[m] is None else _join(entry[m], st)
                if new != entry[m]:
                    entry[m] = new
                    changed = True
    bad = []
    for n, (_, ins) in enumerate(blocks):
        st = entry[n] if entry[n] is not None else {}
        for pos, (in_asm, l) in enumerate(ins):
            op = l.split()[0]
            ops = _operands(l)
            if not op.startswith("v_mfma"):
                # sources: every operand but a VALU's first (its destination); stores and
                # other non-VALU instructions may read an AGPR in any position
                srcs = ops[1:] if op.startswith("v_") else ops
                read = set().union(*(_agprs(t) for t in srcs)) if srcs else set()
                short = sorted(r for r in read if r in st)
                if short:
                    bad.append(f"{l} reads a{short[0]} {st[short[0]]} wait states after an "
                               "MFMA wrote it")
            if in_asm and op.startswith("v_mfma"):
                srcs = set().union(*(_regs(t) for t in ops[1:3]))
                for back in range(1, VALU_TO_ASM_MFMA + 1):
                    if pos - back < 0:
                        break
                    _, prev = ins[pos - back]
                    pop = prev.split()[0]
                    if pop.startswith("v_") and not pop.startswith("v_mfma"):
                        if _regs(_operands(prev)[0]) & srcs:
                            bad.append(f"{l} reads a VGPR {back - 1} instructions after {prev}")
            st = _step(st, l)
    return bad


def check_assembly(text, name_filter):
    """{kernel symbol: violations} for every function whose symbol contains name_filter."""
    s = text.splitlines()
    out = {}
    for k, l in enumerate(s):
        m = re.match(r"^(_ZN\S*):", l)
        if not m or name_filter not in m.group(1):
            continue
        end = next(x for x in range(k, len(s)) if s[x].startswith(".Lfunc_end"))
        out[m.group(1)] = check_function(s[k + 1:end])
    return out
