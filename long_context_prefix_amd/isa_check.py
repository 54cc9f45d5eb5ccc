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
``v_mfma`` it walks every path of instructions that can follow it, counting one
wait state per instruction and N + 1 per ``s_nop N`` (a conditional branch
continues both into the next instruction and at its target, a jump at its
target, so a block that the common path branches over is not counted as
distance), and reports any VALU instruction (``v_accvgpr_read`` included), LDS
or memory store that reads one of the result registers, and any VALU
instruction or load that overwrites one, before ``WAIT_STATES`` have passed on
some path; and, walking back along every path that can lead to the MFMA, any
VALU write of one of its operands fewer than ``OPERAND_WAIT_STATES`` before it.
Using the result as the accumulator of the next MFMA of the same chain is the
one allowed access.
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


_LABEL = re.compile(r"^(\.L\w+):")
_STOP = ("s_endpgm", "s_setpc_b64", "s_trap")


def _is_code(t: str) -> bool:
    return bool(t) and not t.startswith(";") and not t.startswith(".") and not t.endswith(":")


def _branch(t: str):
    """(target label, conditional?) of a branch instruction, else None."""
    op = t.split()[0]
    if op == "s_branch":
        return t.split()[-1], False
    if op.startswith("s_cbranch_"):
        return t.split()[-1], True
    return None


def _cost(t: str) -> int:
    return int(t.split()[1], 0) + 1 if t.split()[0] == "s_nop" else 1


def inline_mfma_hazards(asm: str, wait_states: int = WAIT_STATES) -> List[str]:
    lines = [l.strip() for l in asm.split("\n")]
    labels = {}
    for k, t in enumerate(lines):
        m = _LABEL.match(t)
        if m:
            labels[m.group(1)] = k
    # predecessors of each label line: the branches that target it (the line before it
    # falls through unless it is a jump or an end)
    branches_to = {}
    for k, t in enumerate(lines):
        if _is_code(t):
            b = _branch(t)
            if b and b[0] in labels:
                branches_to.setdefault(labels[b[0]], []).append(k)

    def walk_forward(start: int, dst: set, mfma: str, kernel: str, found: list) -> None:
        best = {}  # line -> fewest wait states it was reached with
        work = [(start, 0)]
        reported = set()
        while work:
            j, ws = work.pop()
            while j < len(lines) and ws < wait_states:
                if best.get(j, wait_states + 1) <= ws:
                    break
                best[j] = ws
                u = lines[j]
                if _KERNEL.match(u):
                    break
                if not _is_code(u):
                    j += 1
                    continue
                op = u.split()[0]
                if op in _STOP:
                    break
                b = _branch(u)
                ws_here = ws + _cost(u)
                if op != "s_nop" and not op.startswith("v_mfma") and b is None:
                    reads, writes = _accesses(u)
                    key = (j, "r" if reads & dst else "w" if writes & dst else "")
                    if key[1] and key not in reported:
                        reported.add(key)
                        what = "reads the result of" if key[1] == "r" else "overwrites the result of"
                        found.append(f"{kernel}: '{u}' {what} '{mfma}' after {ws_here} wait states")
                ws = ws_here
                if b is not None:
                    target, conditional = b
                    if target in labels:
                        work.append((labels[target], ws))
                    if not conditional:
                        break
                j += 1

    def walk_back(start: int, srcs: set, mfma: str, kernel: str, found: list) -> None:
        best = {}
        work = [(start - 1, 0)]
        reported = set()
        while work:
            j, ws = work.pop()
            while j >= 0 and ws < OPERAND_WAIT_STATES:
                if best.get(j, OPERAND_WAIT_STATES + 1) <= ws:
                    break
                best[j] = ws
                u = lines[j]
                if _KERNEL.match(u):
                    break
                if j in branches_to:  # a label line: other paths arrive here too
                    for k in branches_to[j]:
                        work.append((k, ws))
                if not _is_code(u):
                    j -= 1
                    continue
                b = _branch(u)
                if b is not None and not b[1] and j != start - 1:
                    break  # a jump elsewhere: this line is not on a path into the MFMA
                op = u.split()[0]
                if op.startswith("v_") and not op.startswith("v_mfma") and _accesses(u)[1] & srcs:
                    if j not in reported:
                        reported.add(j)
                        found.append(f"{kernel}: '{mfma}' reads an operand written by '{u}' after {ws} wait states")
                ws += _cost(u)
                j -= 1

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
        srcs = set()
        for o in _operands(t)[1:]:
            srcs |= _regs(o)
        walk_back(i, srcs, t, kernel, found)
        walk_forward(i + 1, dst, t, kernel, found)
    return found


# Kernels whose registers must fit without scratch: every bf16 forward and split-KV partial
# kernel (32- and 64-row, fused, partial, merging, mixed).  A spill there moves bytes through
# memory on every launch (at the inducing split-KV shape two 16-byte spills per lane were
# 131 MB of scratch writes per launch).  The fp32 path, kept for correctness only, and the
# backward kernels are not covered.
_NO_SCRATCH = re.compile(r"^_ZN3lcp(15attn_fwd_kernelINS_7Bf16Dma|20attn_fwd_wide_kernel|21attn_fwd_mixed_kernel)")
_KERNEL_DESC = re.compile(r"^\s*\.amdhsa_kernel\s+(\S+)")
_PRIVATE = re.compile(r"^\s*\.amdhsa_private_segment_fixed_size\s+(\d+)")


def private_segment_sizes(asm: str) -> dict:
    """Per-lane scratch bytes of every kernel descriptor in the assembly."""
    sizes = {}
    kernel = None
    for line in asm.split("\n"):
        m = _KERNEL_DESC.match(line)
        if m:
            kernel = m.group(1)
            continue
        m = _PRIVATE.match(line)
        if m and kernel is not None:
            sizes[kernel] = int(m.group(1))
            kernel = None
    return sizes


def scratch_findings(asm: str) -> List[str]:
    """The forward kernels that must not use scratch but do."""
    return [f"{k}: {n} bytes of scratch per lane" for k, n in sorted(private_segment_sizes(asm).items())
            if n > 0 and _NO_SCRATCH.match(k)]
