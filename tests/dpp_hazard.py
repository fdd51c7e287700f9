"""Checks gfx950 assembly for one hazard the compiler does not guard inside
inline asm: a DPP instruction reading (as its swizzled src0) a VGPR that a
VALU instruction wrote fewer than two wait states earlier.  The kernels'
column substitutions issue `v_fmac_f32_dpp` from inline asm, so the wait
states in front of each must come from the surrounding code.

check(asm_text) returns a list of (function, line number, text) for every
DPP instruction with such a write within its two preceding wait states.
"""
import re

_REG = re.compile(r"v\[(\d+):(\d+)\]|v(\d+)\b")


def _regs(operand):
    out = set()
    for m in _REG.finditer(operand):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _operands(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return []
    return [p.strip() for p in parts[1].split(",")]


def _written(line):
    """VGPRs a VALU instruction writes (empty for anything else)."""
    op = line.split(None, 1)[0]
    if not op.startswith("v_"):
        return set()
    ops = _operands(line)
    if not ops:
        return set()
    if op.startswith("v_cmp") or op.startswith("v_readlane") or op.startswith("v_readfirstlane"):
        return set()  # these write SGPRs / VCC
    w = _regs(ops[0])
    if op.startswith("v_permlane16_swap") or op.startswith("v_permlane32_swap") or op.startswith("v_swap"):
        w |= _regs(ops[1])  # both operands are written
    return w


def _wait_states(line):
    op = line.split(None, 1)[0]
    if op == "s_nop":
        ops = _operands(line)
        return int(ops[0], 0) + 1 if ops else 1
    return 1


def check(asm_text):
    bad = []
    func = None
    prev = []  # (line number, text) of the preceding instructions in this function
    for no, raw in enumerate(asm_text.splitlines(), 1):
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":") and not line.startswith("."):
            if not line.startswith(".L") and not line.startswith("$"):
                func = line[:-1]
                prev = []
            else:
                prev.append((no, "<label>"))  # control may arrive from elsewhere
            continue
        if line.startswith("."):
            continue
        op = line.split(None, 1)[0]
        if "_dpp" in op and not op.startswith("v_mov_b32_dpp"):
            src0 = _regs(_operands(line)[1]) if len(_operands(line)) > 1 else set()
            ws = 0
            for pno, ptext in reversed(prev):
                if ptext == "<label>":
                    break
                if _written(ptext) & src0:
                    bad.append((func, no, raw.strip()))
                    break
                ws += _wait_states(ptext)
                if ws >= 2:
                    break
        prev.append((no, line))
        if len(prev) > 64:
            prev = prev[-64:]
    return bad
