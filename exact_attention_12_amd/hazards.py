"""Static check of generated gfx950 assembly for two hazards the compiler does
not track around inline-assembly MFMAs:
  * a VALU write of a register followed, within fewer than two wait states,
    by an MFMA that reads it as an A, B or C operand;
  * an AGPR-accumulating MFMA followed, within fewer than 18 wait states, by
    a VALU instruction that reads or writes its destination (for example a
    copy of the accumulator the register allocator places at a loop
    boundary): the product is still being written. 18 covers the 16-pass
    forms; the 8-pass products used here need fewer.

The compiler inserts these wait states itself around the matrix instructions
it emits, but not around inline-assembly MFMAs (the AGPR-accumulating products
of the dK/dV pass), whose callers separate operand production from the
products with an explicit gap instead. The build runs this check over the
device assembly of every source that uses them and fails on any finding.

Counting follows the ISA's rule: every instruction issued in between is one
wait state, `s_nop N` is N + 1. For the first rule a label inside the window
counts as a finding (another path may reach the MFMA with a closer write);
the second follows the fall-through path up to an unconditional branch.
MFMAs with VGPR destinations are the compiler's own and are not checked by
the second rule (it tracks them itself).
"""

from __future__ import annotations

import re

_REG = re.compile(r"([va])\[(\d+):(\d+)\]$|([va])(\d+)$")
_FUNC = re.compile(r"^(_Z\w+):", re.M)


def _regs(operand: str) -> set:
    m = _REG.match(operand.strip())
    if not m:
        return set()
    if m.group(1):
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {(m.group(4), int(m.group(5)))}


def _operands(line: str) -> list:
    parts = line.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def check(asm: str, wait_states: int = 2, result_wait_states: int = 18) -> list:
    """Findings as (function, [instructions from the first to the second
    instruction of the hazard])."""
    found = []
    for m in _FUNC.finditer(asm):
        name = m.group(1)
        end = asm.find(".Lfunc_end", m.end())
        lines = []
        for raw in asm[m.end():end].splitlines():
            t = raw.split(";")[0].strip()
            if not t or (t.startswith(".") and not t.endswith(":")):
                continue
            lines.append(t)
        for n, line in enumerate(lines):
            if not line.startswith("v_mfma"):
                continue
            ops = _operands(line)
            reads = set().union(*(_regs(o) for o in ops[1:4]))
            ws, k = 0, n - 1
            while k >= 0 and ws < wait_states:
                prev = lines[k]
                if prev.endswith(":"):
                    found.append((name, lines[k:n + 1]))
                    break
                op = prev.split()[0]
                if op == "s_nop":
                    ws += int(prev.split()[1], 0) + 1
                else:
                    if op.startswith("v_") and not op.startswith("v_mfma"):
                        dst = _operands(prev)[:1]
                        if dst and _regs(dst[0]) & reads:
                            found.append((name, lines[k:n + 1]))
                            break
                    ws += 1
                k -= 1
            # second rule: this MFMA's AGPR result read or written too early
            if not ops or not ops[0].startswith("a"):
                continue
            dst = _regs(ops[0])
            ws, k = 0, n + 1
            while k < len(lines) and ws < result_wait_states:
                nxt = lines[k]
                if nxt.endswith(":"):
                    k += 1
                    continue
                op = nxt.split()[0]
                if op == "s_branch" or op == "s_endpgm":
                    break
                if op == "s_nop":
                    ws += int(nxt.split()[1], 0) + 1
                else:
                    if op.startswith("v_") and not op.startswith("v_mfma"):
                        if set().union(*(_regs(o) for o in _operands(nxt))) & dst:
                            found.append((name, lines[n:k + 1]))
                            break
                    ws += 1
                k += 1
    return found
