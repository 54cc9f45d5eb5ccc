"""Static check of the compiled gfx950 assembly: no early access to an inline MFMA result.

Some MFMAs are written as inline assembly so that their accumulators stay in
the register file the kernel wants: the score MFMAs keep their results in VGPRs
(``mfma_vgpr_first`` / ``mfma_vgpr_acc`` in the kernel header) and the O
accumulation of the 64-row D = 256 kernel keeps its accumulator in AGPRs
(``mfma_agpr_acc``).  The compiler does not know those instructions are MFMAs,
so it cannot insert the wait states the hardware needs between an XDL
instruction that writes a register and a later instruction that reads it (or
writes it again).  The kernels leave those wait states by construction; this
check proves it on the actual assembly after every build: for every inline
``v_mfma`` it walks the following instructions, counting one wait state per
instruction and N + 1 per ``s_nop N``, and reports any VALU instruction
(``v_accvgpr_read`` included), LDS or memory store that reads one of the
result registers, and any VALU instruction or load that overwrites one, before
``WAIT_STATES`` have passed, and any VALU write of one of its operands fewer
than ``OPERAND_WAIT_STATES`` before it.  Using the result as the accumulator of
the next MFMA of the same chain is the one allowed access.
"""

from __future__ import annotations

import re
from typing import List

# More than the XDL-write -> VALU-read requirement of any 32x32 MFMA on this target.
WAIT_STATES = 24
# More than the VALU-write -> MFMA-operand-read requirement.
OPERAND_WAIT_STATES = 4

_KERNEL = re.compile(r"^(_Z\S+):")
_RANGE = re.compile(r"([va])\[(\d+):(\d+)\]")
_ONE = re.compile(r"([va])(\d+)$")


def _regs(operand: str) -> set:
    """VGPRs and AGPRs named by one operand, as ('v', n) / ('a', n)."""
    operand = operand.strip()
    m = _RANGE.match(operand)
    if m:
        return {(m.group(1), n) for n in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _ONE.match(operand)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(line: str) -> list:
    _, _, rest = line.partition(" ")
    return [o.split()[0] if o.split() else "" for o in rest.split(",")]


def _accesses(line: str):
    """(registers read, registers written) by one instruction, as far as this check needs."""
    op = line.split()[0]
    ops = _operands(line)
    reads, writes = set(), set()
    if op.startswith("v_"):  # VALU: the first operand is the destination
        writes = _regs(ops[0]) if ops else set()
        for o in ops[1:]:
            reads |= _regs(o)
    elif "_load" in op or op.startswith("ds_read"):
        writes = _regs(ops[0]) if ops else set()  # loads into registers
    elif "_store" in op or op.startswith("ds_write"):
        for o in ops:
            reads |= _regs(o)
    return reads, writes


def inline_mfma_hazards(asm: str, wait_states: int = WAIT_STATES) -> List[str]:
    lines = [l.strip() for l in asm.split("\n")]
    found = []
    kernel = "?"
    in_asm = False
    for i, t in enumerate(lines):
        m = _KERNEL.match(t)
        if m:
            kernel = m.group(1)
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not (in_asm and t.startswith("v_mfma")):
            continue
        parts = t.split(None, 1)
        dst = _regs(parts[1].split(",")[0]) if len(parts) > 1 else set()
        if not dst:
            continue
        # the operands must not have been written by a VALU instruction just before
        srcs = set()
        for o in _operands(t)[1:]:
            srcs |= _regs(o)
        ws = 0
        j = i - 1
        while j >= 0 and ws < OPERAND_WAIT_STATES:
            u = lines[j]
            j -= 1
            if not u or u.startswith(";") or u.startswith(".") or u.endswith(":"):
                continue
            op = u.split()[0]
            if op == "s_nop":
                ws += int(u.split()[1], 0) + 1
                continue
            if op.startswith("v_") and not op.startswith("v_mfma") and _accesses(u)[1] & srcs:
                found.append(f"{kernel}: '{t}' reads an operand written by '{u}' after {ws} wait states")
            ws += 1
        ws = 0
        j = i + 1
        while j < len(lines) and ws < wait_states:
            u = lines[j]
            j += 1
            if not u or u.startswith(";") or u.startswith(".") or u.endswith(":"):
                continue
            op = u.split()[0]
            if op == "s_nop":
                ws += int(u.split()[1], 0) + 1
                continue
            ws += 1
            if op.startswith("v_mfma"):
                continue
            reads, writes = _accesses(u)
            if reads & dst:
                found.append(f"{kernel}: '{u}' reads the result of '{t}' after {ws} wait states")
            elif writes & dst:
                found.append(f"{kernel}: '{u}' overwrites the result of '{t}' after {ws} wait states")
    return found
