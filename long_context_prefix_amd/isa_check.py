"""Static check of the compiled gfx950 assembly: no early read of an inline MFMA result.

Some score MFMAs are written as inline assembly so that their accumulators stay
in VGPRs (see ``mfma_vgpr_first`` / ``mfma_vgpr_acc`` in the kernel header).
The compiler does not know those instructions are MFMAs, so it cannot insert
the wait states the hardware needs between an XDL instruction that writes a
VGPR and a later VALU instruction (or store) that reads it.  The kernels leave
those wait states by construction; this check proves it on the actual
assembly after every build: for every inline ``v_mfma`` with a VGPR result it
walks the following instructions, counting one wait state per instruction and
N + 1 per ``s_nop N``, and reports any VALU instruction, LDS store or memory
store that reads one of the result registers before ``WAIT_STATES`` have
passed.  Reading the result as the accumulator of the next MFMA of the same
chain is the one allowed use.
"""

from __future__ import annotations

import re
from typing import List

# More than the XDL-write -> VALU-read requirement of any 32x32 MFMA on this target.
WAIT_STATES = 24

_KERNEL = re.compile(r"^(_Z\S+):")
_VRANGE = re.compile(r"v\[(\d+):(\d+)\]")
_VONE = re.compile(r"v(\d+)$")


def _vregs(operand: str) -> set:
    operand = operand.strip()
    m = _VRANGE.match(operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = _VONE.match(operand)
    return {int(m.group(1))} if m else set()


def _sources(line: str) -> set:
    op, _, rest = line.partition(" ")
    ops = [o for o in rest.split(",")]
    if op.startswith("v_"):
        ops = ops[1:]  # the first operand of a VALU instruction is its destination
    regs = set()
    for o in ops:
        regs |= _vregs(o.split()[0] if o.split() else "")
    return regs


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
        dst = _vregs(parts[1].split(",")[0]) if len(parts) > 1 else set()
        if not dst:
            continue
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
            reader = op.startswith("v_") or op.startswith("ds_write") or op.startswith("global_store") \
                or op.startswith("buffer_store") or op.startswith("flat_store") or op.startswith("scratch_store")
            if reader and _sources(u) & dst:
                found.append(f"{kernel}: '{u}' reads the result of '{t}' after {ws} wait states")
    return found
