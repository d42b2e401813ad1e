"""Static checks of the backward kernels' generated gfx950 assembly.

The dK/dV and dQ kernels issue their MFMAs as inline assembly (so that long-lived
accumulators stay in AGPRs and score tiles in VGPRs).  The compiler's hazard
recognizer does not look into inline assembly, so two hardware hazards are the
kernels' own responsibility:

* a VALU instruction (including accumulator moves) writing a register that an
  MFMA reads as a source needs two wait states before the MFMA;
* an MFMA result read by another vector instruction needs the MFMA to have
  finished: the kernels keep another MFMA, or enough wait states, in between.

These helpers scan the assembly (``hipcc --cuda-device-only -S``) for both
patterns in the inline-asm MFMAs of the named kernels.
"""
import re

_REG = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)\b")


def regs(tok):
    """Set of (class, index) registers named by one operand."""
    out = set()
    for m in _REG.finditer(tok):
        if m.group(1):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _operands(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.strip() for o in parts[1].split(";")[0].split(",")]


def kernel_bodies(asm_text):
    """{kernel symbol: list of (instruction, inside_inline_asm)}."""
    out = {}
    for m in re.finditer(r"^(_Z\w+):(.*?)\.Lfunc_end", asm_text, re.S | re.M):
        ins, in_asm = [], False
        for raw in m.group(2).split("\n"):
            line = raw.strip()
            if line.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if line.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not line or line.startswith(";") or line.startswith(".") or line.endswith(":"):
                continue
            ins.append((line, in_asm))
        out[m.group(1)] = ins
    return out


def valu_to_mfma_hazards(ins, window=2):
    """Inline-asm MFMAs with a source written by a vector ALU instruction among
    the `window` instructions before it (an s_nop in between ends the search)."""
    found = []
    for k, (line, in_asm) in enumerate(ins):
        if not (in_asm and line.startswith("v_mfma")):
            continue
        ops = _operands(line)
        srcs = set().union(*[regs(o) for o in ops[1:]]) if len(ops) > 1 else set()
        for back in range(1, window + 1):
            if k - back < 0:
                break
            prev = ins[k - back][0]
            if prev.startswith("s_nop"):
                break
            if prev.startswith("v_") and not prev.startswith("v_mfma"):
                pops = _operands(prev)
                if pops and regs(pops[0]) & srcs:
                    found.append((prev, line))
                    break
    return found


def early_result_reads(ins, wait_states=20, wait_states_16=12):
    """Vector instructions reading the result of the last inline-asm MFMA before
    another MFMA issued and before `wait_states` (32x32 shapes, 16 passes) or
    `wait_states_16` (16x16 shapes) wait states (s_nop N counts N+1, any other
    instruction 1)."""
    found = []
    pending, ws, need = set(), 0, wait_states
    for line, in_asm in ins:
        if line.startswith("s_branch") or line.startswith("s_endpgm"):
            pending = set()  # what follows is reached by a jump, not from here
            continue
        if line.startswith("v_mfma"):
            ops = _operands(line)
            pending = regs(ops[0]) if (in_asm and ops) else set()
            need = wait_states if "32x32" in line else wait_states_16
            ws = 0
            continue
        if line.startswith("s_nop"):
            ws += int(line.split()[1]) + 1
        else:
            ops = _operands(line)
            if pending and ws < need and (
                line.startswith("v_") or line.startswith("ds_write") or line.startswith("global_store")
                or line.startswith("buffer_store")
            ):
                srcs = set().union(*[regs(o) for o in ops[1:]]) if len(ops) > 1 else set()
                if srcs & pending:
                    found.append(line)
            if pending and line.startswith("v_") and ops:
                pending -= regs(ops[0])  # overwritten: later reads see the new value
            ws += 1
        if ws >= need:
            pending = set()
    return found
