"""Wait-state checker for MFMAs that the compiler cannot see.

The pipelined backward kernels write their MFMAs as inline assembly, so the
compiler's hazard recognizer does not space the instructions around them.
This module compiles a kernel source to gfx950 assembly and walks every
function in program order, counting wait states (one per instruction,
N + 1 for ``s_nop N``), and reports:

* RAW into an MFMA: a vector ALU write (``v_accvgpr_write`` included) of a
  VGPR or AGPR the MFMA reads, fewer than
  ``SRC_AB`` (A / B operands) or ``SRC_C`` (accumulator input, separate or
  the result registers themselves) wait states before it;
* RAW out of an MFMA: a non-MFMA instruction reading an MFMA result (VGPR or,
  through ``v_accvgpr_read``, AGPR) fewer than ``RESULT`` wait states after
  it; an MFMA that accumulates into the same registers is not a reader;
* WAR on a separate accumulator input: a write to those VGPRs fewer than
  ``SRC_C_WAR`` wait states after the MFMA.

The walk is linear: a forward branch can only make it report more, never
less; a loop's back edge is not followed.
"""

from __future__ import annotations

import os
import re
import subprocess

SRC_AB = 2
SRC_C = 5
RESULT = 19
SRC_C_WAR = 18

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def compile_to_asm(src: str, out: str) -> str:
    from exact_tiled_attention_attn_amd import build as B

    cmd = [B.HIPCC, "-x", "hip", *B.DEVICE, *B.COMMON, "--cuda-device-only", "-S", src, "-o", out]
    if os.path.basename(src) not in B.AGPR_FORM_SOURCES:
        cmd[3:3] = B.VGPR_FORM
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr[-3000:])
    return out


def _regs(tok: str):
    out = set()
    for m in _REG.finditer(tok):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            out.update((kind, r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _split(ins: str):
    parts = ins.split(None, 1)
    op = parts[0]
    args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
    return op, args


def _writes_reads(op: str, args):
    """(registers written, registers read) of a non-MFMA instruction."""
    if not args:
        return set(), set()
    if op.startswith(("ds_write", "buffer_store", "global_store", "flat_store", "scratch_store")):
        return set(), set().union(*[_regs(a) for a in args])
    if op.startswith(("v_", "ds_", "buffer_load", "global_load", "flat_load", "scratch_load")):
        if op.startswith(("v_cmp", "v_cmpx")) and not op.startswith("v_cmp_class"):
            return set(), set().union(*[_regs(a) for a in args])
        w = _regs(args[0])
        r = set().union(*[_regs(a) for a in args[1:]]) if len(args) > 1 else set()
        return w, r
    return set(), set()


def functions(asm: str):
    """{name: [instructions]} of every kernel in an assembly listing."""
    out = {}
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        name = m.group(1)
        end = asm.find(".Lfunc_end", m.end())
        body = asm[m.end():end]
        ins = []
        for line in body.splitlines():
            t = line.split(";")[0].strip()
            if not t or t.startswith(".") or t.endswith(":"):
                continue
            ins.append(t)
        out[name] = ins
    return out


def m0_writers(ins):
    """Instructions writing M0 that are not an s_mov_b32 followed by s_nop 0 (set_m0)."""
    out = []
    for i, t in enumerate(ins):
        op, args = _split(t)
        if args and args[0] == "m0" and not (op == "s_mov_b32" and i + 1 < len(ins) and ins[i + 1] == "s_nop 0"):
            out.append(t)
    return out


def check(ins):
    """List of hazard descriptions for one function's instructions."""
    problems = []
    ws = []  # wait-state position of each instruction
    pos = 0
    for t in ins:
        op, args = _split(t)
        ws.append(pos)
        pos += int(args[0]) + 1 if op == "s_nop" and args else 1
    for i, t in enumerate(ins):
        op, args = _split(t)
        if not op.startswith("v_mfma"):
            continue
        dst = _regs(args[0])
        srcab = _regs(args[1]) | _regs(args[2])
        srcc = _regs(args[3]) if len(args) > 3 else set()
        separate_c = bool(srcc) and srcc != dst
        # RAW into the MFMA.
        for j in range(i - 1, -1, -1):
            gap = ws[i] - ws[j]
            if gap >= max(SRC_AB, SRC_C):
                break
            pop, pargs = _split(ins[j])
            if not pop.startswith("v_") or pop.startswith("v_mfma"):
                continue
            w, _ = _writes_reads(pop, pargs)
            if gap < SRC_AB and w & srcab:
                problems.append(f"{ins[j]} -> {t}: A/B operand {gap} wait states after a vector write")
            if gap < SRC_C and w & srcc:
                problems.append(f"{ins[j]} -> {t}: accumulator input {gap} wait states after a vector write")
        # After the MFMA: reads of its result, writes of a separate accumulator input.
        for j in range(i + 1, len(ins)):
            gap = ws[j] - ws[i]
            if gap >= max(RESULT, SRC_C_WAR):
                break
            nop, nargs = _split(ins[j])
            if nop.startswith("v_mfma"):
                ndst = _regs(nargs[0])
                nsrc = _regs(nargs[1]) | _regs(nargs[2])
                if gap < RESULT and nsrc & dst:
                    problems.append(f"{t} -> {ins[j]}: result read as an A/B operand {gap} wait states later")
                if ndst & dst and not (len(nargs) > 3 and _regs(nargs[3]) == dst == ndst):
                    if gap < RESULT:
                        problems.append(f"{t} -> {ins[j]}: result overwritten {gap} wait states later")
                continue
            w, r = _writes_reads(nop, nargs)
            if gap < RESULT and r & dst:
                problems.append(f"{t} -> {ins[j]}: result read {gap} wait states later")
            if separate_c and gap < SRC_C_WAR and w & {x for x in srcc if x[0] == "v"}:
                problems.append(f"{t} -> {ins[j]}: accumulator input overwritten {gap} wait states later")
    return problems
