"""Wait-state checks on generated gfx950 code for the instructions the 64-query-wave kernel
writes as inline asm (the compiler's hazard recognizer does not look inside inline asm):

  * an MFMA with an AGPR accumulator must be >= 2 wait states after a VALU write of any of
    its sources;
  * no non-MFMA instruction may touch such an MFMA's accumulator within 12 wait states after
    it (16 are issued);
  * an ordinary VALU read of a v_dot2c result must be >= 3 wait states after it (a following
    v_dot2c accumulating into it is fine);
  * write after read: a VALU write of a VGPR that an MFMA reads as its accumulator input
    (SrcC in VGPRs, not also its destination) must wait until the MFMA has read it over all
    its passes (16 wait states is taken as the bound here). A VALU write of a register the MFMA reads as SrcA or SrcB
    needs no wait states: the ISA's MFMA dependency table lists write-after-read only for
    SrcC, A and B being read when the MFMA issues. The compiler's own schedules rely on this
    (compiler_source_war_pairs counts the places where it writes an A/B register in the very
    next instruction), so the rule is taken from the toolchain, not from a probe of the chip.

Each instruction counts one wait state, s_nop N counts N + 1. Linear scan per kernel
(labels are fall-through)."""
import re


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _parse(line):
    t = line.strip()
    if not t or t.startswith((";", ".")) or t.endswith(":"):
        return None
    t = t.split(";")[0].strip()
    parts = t.split(None, 1)
    ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
    return parts[0], ops


def _insts(lines):
    """[(opcode, operands, inside inline asm)] for one kernel's lines."""
    out, in_asm = [], False
    for l in lines:
        if "ASMSTART" in l:
            in_asm = True
        elif "ASMEND" in l:
            in_asm = False
        else:
            p = _parse(l)
            if p:
                out.append((p[0], p[1], in_asm))
    return out


def _is_valu_write(op, ops):
    return op.startswith("v_") and not op.startswith("v_mfma") and bool(ops)


def compiler_source_war_pairs(lines):
    """Number of compiler-generated MFMAs whose next instruction (also compiler-generated) is
    a VALU write of one of the MFMA's SrcA/SrcB registers."""
    insts = _insts(lines)
    n = 0
    for i in range(len(insts) - 1):
        op, ops, asm = insts[i]
        if asm or not op.startswith("v_mfma") or len(ops) < 3:
            continue
        nop, nops, nasm = insts[i + 1]
        if not nasm and _is_valu_write(nop, nops) and \
                _regs(nops[0]) & set().union(*(_regs(o) for o in ops[1:3])):
            n += 1
    return n


def check_kernel(lines):
    """Returns a list of hazard descriptions for one kernel's instruction lines."""
    insts = [(op, ops) for op, ops, _ in _insts(lines)]
    bad = []
    for i, (op, ops) in enumerate(insts):
        if op.startswith("v_mfma") and len(ops) >= 4 and ops[3].startswith("v"):
            src_c = _regs(ops[3]) - _regs(ops[0])   # an in-place accumulator is a result read
            ws = 0
            for j in range(i + 1, min(len(insts), i + 40)):
                pop, pops = insts[j]
                if pop == "s_nop":
                    ws += int(pops[0]) + 1
                    continue
                if ws >= 16:
                    break
                if _is_valu_write(pop, pops) and _regs(pops[0]) & src_c:
                    bad.append(f"{op} reads {ops[3]} as SrcC, then {pop} writes {pops[0]}")
                ws += 1
        if op.startswith("v_mfma") and ops and ops[0].startswith("a["):
            srcs = set().union(*(_regs(o) for o in ops[1:]))
            ws = 0
            for j in range(i - 1, max(-1, i - 8), -1):
                pop, pops = insts[j]
                if pop == "s_nop":
                    ws += int(pops[0]) + 1
                    continue
                if ws >= 2:
                    break
                if pop.startswith("v_") and not pop.startswith("v_mfma") and pops and _regs(pops[0]) & srcs:
                    bad.append(f"VALU write {pop} {pops[0]} then {op} {','.join(ops)}")
                ws += 1
            dst = _regs(ops[0])
            ws = 0
            for j in range(i + 1, min(len(insts), i + 40)):
                pop, pops = insts[j]
                if pop == "s_nop":
                    ws += int(pops[0]) + 1
                    continue
                if ws >= 12:
                    break
                if not pop.startswith("v_mfma") and pops and set().union(*(_regs(o) for o in pops)) & dst:
                    bad.append(f"{op} {ops[0]} then {pop} {','.join(pops)}")
                ws += 1
        if op.startswith("v_dot2c") and ops:
            dst = _regs(ops[0])
            ws = 0
            for j in range(i + 1, min(len(insts), i + 10)):
                pop, pops = insts[j]
                if pop == "s_nop":
                    ws += int(pops[0]) + 1
                    continue
                if ws >= 3:
                    break
                if pop.startswith("v_") and not pop.startswith("v_dot2c") and len(pops) > 1 and \
                        set().union(*(_regs(o) for o in pops[1:])) & dst:
                    bad.append(f"{op} {ops[0]} then {pop} {','.join(pops)}")
                ws += 1
    return bad


def check_asm(text):
    """{kernel name: [hazards]} for every kernel symbol in an assembly listing."""
    out, name, cur = {}, None, []
    for l in text.splitlines():
        m = re.match(r"^(_Z\w+):", l)
        if m:
            if name:
                out[name] = check_kernel(cur)
            name, cur = m.group(1), []
        elif name:
            if l.startswith(".Lfunc_end"):
                out[name] = check_kernel(cur)
                name, cur = None, []
            else:
                cur.append(l)
    if name:
        out[name] = check_kernel(cur)
    return out
