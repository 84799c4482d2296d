"""Checks of the device code of a linked libfa.so (CPU only, llvm-objdump).

``build()`` runs ``check_library`` on the freshly linked library and refuses to
install it when a check fails; ``tests/test_device_code.py`` runs the same checks
on the installed one and tests the scanner itself.

1. Wait states before the LDS-direct buffer loads.  The 16-bit kernels copy
   tiles with `buffer_load_dword{,x4} ... offen lds`, issued as inline assembly.
   The compiler's hazard recognizer does not look inside inline assembly, so
   the wait states the hardware needs before such a load are the copy helper's
   own business:

     * a VALU write of an SGPR (v_readlane of a spilled descriptor,
       v_readfirstlane, the SGPR result of a compare or carry) needs 5 wait
       states before a VMEM instruction reads that SGPR (the descriptor, the
       soffset, M0);
     * a SALU write of M0 needs 1 wait state before a load that writes LDS.

   A load that reads its descriptor too early takes stale SGPRs as the base
   address: a build whose dK/dV dropout instance reloaded the descriptor with
   v_readlane right before the copy faulted with an illegal address.  Every
   gfx950 code object of the library is disassembled and the instructions
   before each such load are checked (a straight-line scan back from the load;
   a branch target inside the window counts as a violation unless the wait
   states up to it suffice).

2. One definition per kernel.  Kernels are templates, so their host-side
   handles are weak symbols: an object file of an older source linked into
   the library would silently supply some of them, compiled against an older
   argument layout.  No kernel may appear in two code objects.

3. Wait states before the MFMAs.  Some kernels issue MFMAs with AGPR
   accumulators as inline assembly, which the hazard recognizer does not see
   either: an MFMA must not read a VGPR (as A, B or C) sooner than two wait
   states after a VALU instruction other than a dot product wrote it, or it
   may read the old value.  Every MFMA of the library is checked (those the
   compiler issued pass by construction).
"""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
import tempfile

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

VALU_SGPR_TO_VMEM = 5
SALU_M0_TO_LDS_DMA = 1

_NAMED = {"vcc": {106, 107}, "vcc_lo": {106}, "vcc_hi": {107}, "m0": {"m0"}}


def sgprs(tok: str) -> set:
    tok = tok.strip()
    if tok in _NAMED:
        return set(_NAMED[tok])
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m[1]), int(m[2]) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    return {int(m[1])} if m else set()


# VALU opcodes whose e64 form has an SGPR destination after the VGPR one (carry
# or flags), and whose e32 form writes VCC.
_CARRY = ("v_add_co_", "v_sub_co_", "v_subrev_co_", "v_addc_co_", "v_subb_co_", "v_subbrev_co_",
          "v_mad_u64_u32", "v_mad_i64_i32", "v_div_scale_")


def writes(ins: str):
    """('valu' | 'salu' | 'other', set of SGPRs (and 'm0') the instruction writes)."""
    op, _, rest = ins.partition(" ")
    ops = [o.strip() for o in rest.split(",")] if rest else []
    if op.startswith("v_"):
        # A VALU destination that is an SGPR comes first (v_readlane,
        # v_readfirstlane, compares in VOP3 or SDWA form); compares in VOPC form
        # write VCC; carry-outs come second.
        out = sgprs(ops[0]) if ops else set()
        if op.startswith("v_cmp") and not out:
            out = set(_NAMED["vcc"])
        elif op.startswith(_CARRY):
            out |= sgprs(ops[1]) if op.endswith("_e64") or "_e" not in op[-4:] else _NAMED["vcc"]
        return "valu", out
    if op.startswith("s_") and ops and not op.startswith(("s_cmp", "s_bitcmp", "s_waitcnt", "s_nop",
                                                         "s_barrier", "s_branch", "s_cbranch")):
        return "salu", sgprs(ops[0])
    return "other", set()


def wait_states(ins: str) -> int:
    m = re.match(r"s_nop\s+(0x[0-9a-fA-F]+|\d+)", ins)
    return int(m[1], 0) + 1 if m else 1


DMA = re.compile(r"buffer_load_\w+\s+v\d+,\s*(s\[\d+:\d+\]),\s*(\w+)\s.*\blds\b")


def violations(lines, targets=frozenset()):
    """(line index, load, offending instruction, wait states between) for every
    LDS-direct buffer load with too few wait states after a write of one of its
    SGPR operands or of M0.  `lines` are bare instructions, None at a function
    start; `targets` the indices of branch targets: control may reach them from
    elsewhere, so a window that reaches back past one is a violation unless the
    wait states counted up to it suffice."""
    out = []
    for i, ins in enumerate(lines):
        m = DMA.match(ins) if ins else None
        if not m:
            continue
        reads = sgprs(m[1]) | sgprs(m[2]) | {"m0"}
        ws = 0
        for j in range(i - 1, -1, -1):
            prev = lines[j]
            if prev is None:       # start of a function
                break
            if j + 1 in targets:
                out.append((i, ins, "a branch target", ws))
                break
            kind, w = writes(prev)
            if kind == "valu" and w & reads and ws < VALU_SGPR_TO_VMEM:
                out.append((i, ins, prev, ws))
                break
            if kind == "salu" and "m0" in w and ws < SALU_M0_TO_LDS_DMA:
                out.append((i, ins, prev, ws))
                break
            ws += wait_states(prev)
            if ws >= VALU_SGPR_TO_VMEM:
                break
    return out


VALU_VGPR_TO_MFMA = 2


def vgprs(tok: str) -> set:
    tok = tok.strip()
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m[1]), int(m[2]) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m[1])} if m else set()


def valu_vgpr_writes(ins: str) -> set:
    """VGPRs a VALU instruction other than an MFMA or a dot product writes (its
    first operand; compares and lane reads write SGPRs)."""
    op, _, rest = ins.partition(" ")
    if not op.startswith("v_") or op.startswith(("v_mfma", "v_dot", "v_cmp", "v_readlane",
                                                 "v_readfirstlane")):
        return set()
    ops = [o.strip() for o in rest.split(",")] if rest else []
    return vgprs(ops[0]) if ops else set()


MFMA = re.compile(r"v_mfma\w*\s+(\S+),\s*(\S+),\s*(\S+),\s*(\S+)")


def mfma_violations(lines, targets=frozenset()):
    """(line index, MFMA, offending instruction, wait states between) for every
    MFMA that reads a VGPR fewer than VALU_VGPR_TO_MFMA wait states after a
    VALU write of it.  `targets` maps each branch target to the lines of the
    branches that reach it; the scan back from an MFMA follows those branches
    as well as the fall-through.  A target whose branches are not known (a
    set) counts as a violation."""
    out = []

    def scan(i, ins, reads, j, ws, depth):
        # Instructions j, j - 1, ... precede the MFMA, ws wait states already
        # between.  Returns the offending instruction, or None.
        while j >= 0 and ws < VALU_VGPR_TO_MFMA:
            prev = lines[j]
            if prev is None:
                return None
            if valu_vgpr_writes(prev) & reads:
                return prev
            ws += wait_states(prev)
            if j in targets and ws < VALU_VGPR_TO_MFMA:
                srcs = targets[j] if isinstance(targets, dict) else None
                if srcs is None or depth > 8:
                    return "a branch target"
                for b in srcs:
                    hit = scan(i, ins, reads, b, ws, depth + 1)
                    if hit:
                        return hit
                if j > 0 and lines[j - 1] and lines[j - 1].startswith("s_branch"):
                    return None   # no fall-through into the target
            j -= 1
        return None

    for i, ins in enumerate(lines):
        m = MFMA.match(ins) if ins else None
        if not m:
            continue
        reads = vgprs(m[2]) | vgprs(m[3]) | vgprs(m[4])
        if i in targets:
            # The MFMA itself is a branch target: check its other entries too.
            srcs = targets[i] if isinstance(targets, dict) else None
            hit = "a branch target" if srcs is None else next(
                (h for b in srcs for h in [scan(i, ins, reads, b, 0, 1)] if h), None)
            if hit:
                out.append((i, ins, hit, 0))
                continue
            if i > 0 and lines[i - 1] and lines[i - 1].startswith("s_branch"):
                continue
        hit = scan(i, ins, reads, i - 1, 0, 0)
        if hit:
            out.append((i, ins, hit, None))
    return out


def code_objects(lib_path: str, workdir: str):
    """Disassembly of every gfx950 code object in the library: a list of
    (function names, bare instructions with None at each function start,
    {index of a branch target: indices of the branches to it}).  `workdir` receives the unbundled objects."""
    lib = os.path.join(workdir, "libfa.so")
    shutil.copy(lib_path, lib)
    subprocess.run([OBJDUMP, "--offloading", lib], cwd=workdir, check=True, capture_output=True)
    objs = sorted(glob.glob(os.path.join(workdir, "libfa.so.*gfx950")))
    if not objs:
        raise RuntimeError(f"no gfx950 code object in {lib_path}")
    out = []
    for obj in objs:
        dis = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", obj], check=True,
                             capture_output=True, text=True).stdout
        names, lines, start, addr, branch, branch_line = [], [], {}, {}, [], []
        for raw in dis.splitlines():
            m = re.match(r"^([0-9a-fA-F]+) <(.*)>:$", raw)
            if m:
                names.append(m[2])
                start[m[2]] = int(m[1], 16)
                lines.append(None)
                continue
            ins = raw.split("//")[0].strip()
            if ins and not ins.endswith(":") and raw[:1] in ("\t", " "):
                a = re.search(r"//\s*([0-9a-fA-F]+):", raw)
                if a:
                    addr[int(a[1], 16)] = len(lines)
                t = re.search(r"<(\S+)\+0x([0-9a-fA-F]+)>\s*$", raw)
                if ins.startswith(("s_branch", "s_cbranch")) and t:
                    branch.append((t[1], int(t[2], 16)))
                    branch_line.append(len(lines))
                lines.append(ins)
        missing = [(f, off) for f, off in branch if f in start and start[f] + off not in addr]
        if missing:
            raise RuntimeError(f"branch targets that start no parsed instruction: {missing[:3]}")
        targets = {}
        for (f, off), src in zip(branch, branch_line):
            if f in start:
                targets.setdefault(addr[start[f] + off], []).append(src)
        out.append((names, lines, targets))
    return out


def function_at(names, lines, i):
    """Name of the function whose code holds line i (lines hold None at each
    function start, in the order of `names`)."""
    k = sum(1 for x in lines[:i + 1] if x is None)
    return names[k - 1] if k else "?"


def kernels_in_several_objects(objs):
    seen = {}
    for i, (names, _, _) in enumerate(objs):
        for n in names:
            if n.startswith("_ZN2fa"):
                seen.setdefault(n, set()).add(i)
    return sorted(n for n, s in seen.items() if len(s) > 1)


def dma_loads(objs) -> int:
    return sum(1 for _, lines, _ in objs for ins in lines if ins and DMA.match(ins))


def check_library(lib_path: str) -> dict:
    """Runs both checks on a linked library.  Returns counts; raises
    RuntimeError naming the first offenders when a check fails, or when the
    disassembly looks unparsed (too few loads, kernels or branch targets)."""
    with tempfile.TemporaryDirectory(prefix="fa_devcheck_") as tmp:
        objs = code_objects(lib_path, tmp)
    n = dma_loads(objs)
    kernels = sum(1 for names, _, _ in objs for x in names if x.startswith("_ZN2fa"))
    if n < 1000 or kernels < 50 or sum(len(t) for _, _, t in objs) < 100:
        raise RuntimeError(f"device-code check: disassembly not parsed ({n} LDS-direct loads, "
                           f"{kernels} kernels)")
    bad = [(function_at(names, lines, v[0]),) + v for names, lines, targets in objs
           for v in violations(lines, targets)]
    if bad:
        where = sorted({f for f, *_ in bad})
        raise RuntimeError(
            f"device-code check: {len(bad)} of {n} LDS-direct loads too soon after an SGPR/M0 "
            f"write, in {where}; e.g. " + "; ".join(f"{p!r} {w} wait states before {ins!r}"
                                                     for _, _, ins, p, w in bad[:4]))
    bad = [(function_at(names, lines, v[0]),) + v for names, lines, targets in objs
           for v in mfma_violations(lines, targets)]
    if bad:
        where = sorted({f for f, *_ in bad})
        raise RuntimeError(
            f"device-code check: {len(bad)} MFMAs read a VGPR too soon after a VALU write, in "
            f"{where}; e.g. " + "; ".join(f"{p!r} {w} wait states before {ins!r}"
                                          for _, _, ins, p, w in bad[:4]))
    dup = kernels_in_several_objects(objs)
    if dup:
        raise RuntimeError(f"device-code check: {len(dup)} kernels defined in more than one code "
                           f"object, e.g. {dup[:3]}")
    return {"lds_dma_loads": n, "kernels": kernels}
