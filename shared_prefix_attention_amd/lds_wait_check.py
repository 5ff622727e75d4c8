"""Build-time check of the hand-placed LDS read waits in the HIP kernels.

The attention kernels issue some LDS reads as inline asm (ds_read_b128 and
the gfx950 transpose reads ds_read_b64_tr_b16 / _b8), so that the compiler
neither waits for in-flight LDS DMA before them nor interleaves them with
their consumers. The compiler does not know such a read is asynchronous: it
takes the destination register as written when the asm statement ends. The
kernels therefore wait by hand (an explicit ``s_waitcnt lgkmcnt(0)`` whose
asm statement takes the destination registers as operands) before any use.

That is sound only while no instruction between the read and the wait
touches the destination registers (a copy, a spill, a reuse of a register
the compiler thinks is free) and no later read's address register is still
in flight. This module verifies exactly that on the compiler's own gfx950
assembly of this library: per kernel, a data-flow pass over the basic blocks
tracks the registers of inline-asm LDS reads not yet covered by an
``lgkmcnt(0)`` wait and reports every instruction that reads or writes one.
Compiler-generated LDS reads are left out: the compiler inserts their waits
itself, and since LDS operations complete in order, extra reads in flight
only make its counted waits stronger.
"""

from __future__ import annotations

import re
from typing import Dict, List, Tuple

TRACKED = ("ds_read_b128", "ds_read_b64_tr_b16", "ds_read_b64_tr_b8", "ds_read_b64", "ds_read_b32")
_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")
_BRANCH_END = ("s_branch", "s_endpgm", "s_setpc_b64")


def _regs(tok: str):
    out = set()
    for m in _REG.finditer(tok):
        if m.group(1):
            out.update((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _functions(text: str) -> Dict[str, list]:
    funcs: Dict[str, list] = {}
    cur = None
    in_asm = False
    for ln, raw in enumerate(text.splitlines(), 1):
        st = raw.strip()
        if st.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if st.startswith(";;#ASMEND"):
            in_asm = False
            continue
        code = st.split(";")[0].strip()
        if not code:
            continue
        m = re.match(r"^([A-Za-z_.$][\w.$]*):", raw)
        if m and not raw.startswith(("\t", " ")):
            name = m.group(1)
            if not name.startswith("."):
                cur = funcs.setdefault(name, [])
            elif cur is not None:
                cur.append(("label", name, ln, False))
            continue
        if code.startswith(".") or cur is None:
            continue
        cur.append(("inst", code, ln, in_asm))
    return funcs


def _check_function(items) -> Tuple[int, Dict[int, str]]:
    blocks: List[list] = [["<entry>", []]]
    label_at: Dict[str, int] = {}
    for kind, x, ln, asm in items:
        if kind == "label":
            blocks.append([x, []])
            label_at[x] = len(blocks) - 1
            continue
        blocks[-1][1].append((x, ln, asm))
        op = x.split()[0]
        if op.startswith("s_cbranch") or op in _BRANCH_END:
            blocks.append([None, []])
    succ = []
    for i, (_, ins) in enumerate(blocks):
        s = []
        last = ins[-1][0] if ins else ""
        op = last.split()[0] if last else ""
        if (op.startswith("s_cbranch") or op == "s_branch") and len(last.split()) > 1:
            tgt = last.split()[1]
            if tgt in label_at:
                s.append(label_at[tgt])
        if op not in _BRANCH_END and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    pending_in = [frozenset() for _ in blocks]
    viol: Dict[int, str] = {}
    reads = 0
    changed = True
    while changed:
        changed = False
        outs = []
        reads = 0
        for i, (_, ins) in enumerate(blocks):
            pend = set(pending_in[i])
            for x, ln, asm in ins:
                parts = x.split(None, 1)
                op, args = parts[0], (parts[1] if len(parts) > 1 else "")
                if op == "s_waitcnt":
                    if "lgkmcnt(0)" in args:
                        pend = set()
                    continue
                ops = [a.strip() for a in args.split(",")] if args else []
                if asm and op in TRACKED:
                    reads += 1
                    src = set().union(*(_regs(a) for a in ops[1:])) if len(ops) > 1 else set()
                    if src & pend:
                        viol[ln] = f"{op}: its address register is the destination of a read still in flight"
                    dst = _regs(ops[0]) if ops else set()
                    if dst & pend:
                        viol[ln] = f"{op}: its destination is still the target of a read in flight"
                    pend |= dst
                    continue
                used = set().union(*(_regs(a) for a in ops)) if ops else set()
                hit = used & pend
                if hit:
                    viol[ln] = f"{op} touches {sorted(hit)[:4]} before its LDS read is waited for"
            outs.append(frozenset(pend))
        new_in = [set() for _ in blocks]
        for i, s in enumerate(succ):
            for j in s:
                new_in[j] |= outs[i]
        for j in range(len(blocks)):
            f = frozenset(new_in[j])
            if f != pending_in[j]:
                pending_in[j] = f
                changed = True
    return reads, viol


def check(asm_text: str) -> Tuple[int, int, List[str]]:
    """Returns (kernels, inline LDS reads, violations) for gfx950 assembly."""
    funcs = _functions(asm_text)
    total = 0
    problems: List[str] = []
    for name, items in funcs.items():
        n, viol = _check_function(items)
        total += n
        problems += [f"{name} line {ln}: {msg}" for ln, msg in sorted(viol.items())]
    return len(funcs), total, problems
