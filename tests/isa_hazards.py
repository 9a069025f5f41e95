"""Check the gfx950 ISA the compiler produced for the bf16 kernel around the
score MFMAs written as inline asm.

The compiler pads hazards for the instructions it emits itself but cannot see
into inline asm.  The kernel relies on every asm MFMA reading only (a) registers
written by an LDS load (waited for by s_waitcnt), (b) the Q operands written into
AGPRs once, long before, and (c) its own chain accumulator.  A vector-ALU write to
one of its source registers in the few instructions before it would need wait
states nobody inserted.  This module finds such writes; registers overwritten by
an MFMA or a memory load into registers in between do not count (the value then
comes from that instruction, whose completion s_waitcnt or the MFMA interlock
orders).
"""
from __future__ import annotations

import re

WINDOW = 6      # instructions scanned back from each asm MFMA


def _regs(tok: str) -> set[str]:
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok) or re.match(r"([va])(\d+)$", tok)
    if not m:
        return set()
    lo = int(m.group(2))
    hi = int(m.group(3)) if m.lastindex == 3 else lo
    return {f"{m.group(1)}{i}" for i in range(lo, hi + 1)}


AFTER_STATES = 18   # wait states after a 32x32 MFMA before anything else may touch its result


def _instructions(asm_text: str):
    """(opcode, operands, inside inline asm) for every instruction line."""
    inasm = False
    for raw in asm_text.split("\n"):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if s.startswith(";;#ASMEND"):
            inasm = False
            continue
        if not s or s.startswith(";") or s.endswith(":") or s.startswith("."):
            continue
        op = s.split()[0]
        yield op, [o.strip() for o in s[len(op):].split(",") if o.strip()], inasm, s


def _loads_into_registers(op: str, ops: list[str]) -> bool:
    """A memory load whose first operand is its destination: LDS, global, scratch
    or buffer loads, except the direct-to-LDS buffer form (its first operand is an
    address)."""
    if op.startswith(("ds_read", "global_load", "scratch_load", "flat_load")):
        return True
    return op.startswith("buffer_load") and not any(o.split()[-1] == "lds" or o.endswith(" lds") for o in ops)


def check(asm_text: str) -> tuple[int, list[str]]:
    """Return (asm MFMAs checked, list of suspicious findings).

    Before an asm MFMA: no vector-ALU write to one of its sources in the WINDOW
    preceding instructions (unless an MFMA rewrote that register in between).
    After it: until AFTER_STATES wait states have passed (each instruction counts
    one, s_nop k counts k + 1), no instruction other than an MFMA accumulating into
    the same registers may read or write its destination."""
    ins = list(_instructions(asm_text))
    found: list[str] = []
    n = 0
    for idx, (op, ops, inasm, text) in enumerate(ins):
        if not (inasm and op.startswith("v_mfma")):
            continue
        n += 1
        live = set().union(*[_regs(o) for o in ops[1:]])
        for pop, pops, _, ptext in reversed(ins[max(0, idx - WINDOW):idx]):
            if not pops:
                continue
            dst = _regs(pops[0])
            if pop.startswith("v_mfma"):
                live -= dst              # value now comes from that MFMA
                continue
            if _loads_into_registers(pop, pops):
                live -= dst              # value now comes from that load
                continue
            if pop.startswith("v_") and dst & live:
                found.append(f"before: {ptext} -> {text}")
        dst = _regs(ops[0])
        states = 0
        for nop, nops, _, ntext in ins[idx + 1:]:
            if states >= AFTER_STATES:
                break
            if nop.startswith("s_nop"):
                states += int(nops[0], 0) + 1 if nops else 1
                continue
            states += 1
            touched = set().union(*[_regs(o) for o in nops]) if nops else set()
            if nop.startswith("v_mfma") and nops and _regs(nops[0]) == dst and _regs(nops[-1]) == dst:
                break                    # the chain continues into the same accumulator
            if touched & dst:
                found.append(f"after: {text} -> {ntext}")
                break
    return n, found
