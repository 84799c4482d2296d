"""Checks of the device code in the built library (no GPU).

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
   gfx950 code object of libfa.so is disassembled and the instructions before
   each such load are checked (a straight-line scan back from the load).

2. One definition per kernel.  Kernels are templates, so their host-side
   handles are weak symbols: an object file of an older source linked into
   the library would silently supply some of them, compiled against an older
   argument layout.  No kernel may appear in two code objects."""
import glob
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "io_aware_exact_fa_amd", "libfa.so")
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


_DMA = re.compile(r"buffer_load_\w+\s+v\d+,\s*(s\[\d+:\d+\]),\s*(\w+)\s.*\blds\b")


def violations(lines, targets=frozenset()):
    """(line index, load, offending instruction, wait states between) for every
    LDS-direct buffer load with too few wait states after a write of one of its
    SGPR operands or of M0.  `lines` are bare instructions, None at a function
    start; `targets` the indices of branch targets: control may reach them from
    elsewhere, so a window that reaches back past one is a violation unless the
    wait states counted up to it suffice."""
    out = []
    for i, ins in enumerate(lines):
        m = _DMA.match(ins) if ins else None
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


def code_objects(tmp_path, lib_path=LIB):
    """Disassembly of every gfx950 code object in the library: a list of
    (function names, bare instructions with None at each function start)."""
    lib = tmp_path / "libfa.so"
    shutil.copy(lib_path, lib)
    subprocess.run([OBJDUMP, "--offloading", str(lib)], cwd=tmp_path, check=True,
                   capture_output=True)
    objs = sorted(glob.glob(str(tmp_path / "libfa.so.*gfx950")))
    assert objs, "no gfx950 code object in libfa.so"
    out = []
    for obj in objs:
        dis = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", obj], check=True,
                             capture_output=True, text=True).stdout
        names, lines, start, addr, branch = [], [], {}, {}, []
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
                lines.append(ins)
        missing = [(f, off) for f, off in branch if f in start and start[f] + off not in addr]
        assert not missing, f"branch targets that start no parsed instruction: {missing[:3]}"
        targets = frozenset(addr[start[f] + off] for f, off in branch if f in start)
        out.append((names, lines, targets))
    return out


def kernels_in_several_objects(objs):
    seen = {}
    for i, (names, _, _) in enumerate(objs):
        for n in names:
            if n.startswith("_ZN2fa"):
                seen.setdefault(n, set()).add(i)
    return sorted(n for n, s in seen.items() if len(s) > 1)


def test_scanner_flags_the_hazards():
    """The scan catches a descriptor reloaded by v_readlane right before the
    copy (the faulting pattern), a carry-out SGPR pair, VCC from an e32 compare
    used as soffset, and M0 set by the instruction before; five wait states
    (s_nop 4) clear the first three and any instruction in between the last."""
    load = "buffer_load_dword v173, s[0:3], s94 offen lds"
    assert violations(["v_readlane_b32 s3, v238, 58", load])
    assert violations(["v_mad_u64_u32 v[174:175], s[0:1], v166, s23, 0", "s_nop 1", load])
    assert violations(["v_cmp_eq_u32_e32 vcc, 0, v1",
                       "buffer_load_dwordx4 v186, s[48:51], vcc_lo offen lds"])
    assert violations(["s_add_i32 m0, s11, 0x5000", load])
    assert not violations(["v_readlane_b32 s3, v238, 58", "s_nop 4", load])
    assert not violations(["v_mad_u64_u32 v[174:175], s[0:1], v166, s23, 0", "s_nop 4", load])
    assert not violations(["s_add_i32 m0, s11, 0x5000", "s_nop 0", load])
    assert not violations(["v_readlane_b32 s7, v238, 58", load])      # another SGPR
    assert not violations([None, load])
    assert violations(["s_nop 4", "s_nop 0", load], targets={1})     # reached by a branch
    assert not violations(["s_nop 0", "s_nop 4", load], targets={1})
    assert violations(["v_cmp_eq_u32_sdwa s[0:1], v1, v2 src0_sel:WORD_0", "s_nop 1", load])
    assert not violations(["v_add_u32_e32 v1, s3, v2", load])          # an SGPR source only
    assert not violations(["s_mov_b32 s3, 0", load])                  # SALU -> VMEM: no wait


@pytest.mark.skipif(not os.path.exists(LIB), reason="libfa.so not built")
@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump not installed")
def test_every_lds_dma_load_has_its_wait_states(tmp_path):
    objs = code_objects(tmp_path)
    n = sum(1 for _, lines, _ in objs for ins in lines if ins and _DMA.match(ins))
    assert n > 1000, f"only {n} LDS-direct loads found: the disassembly was not parsed"
    assert sum(len(t) for _, _, t in objs) > 100, "no branch targets found"
    bad = [v for _, lines, targets in objs for v in violations(lines, targets)]
    assert not bad, f"{len(bad)} of {n} LDS-direct loads too soon after an SGPR/M0 write, e.g. " + \
        "; ".join(f"{p!r} {w} wait states before {ins!r}" for _, ins, p, w in bad[:4])


@pytest.mark.skipif(not os.path.exists(LIB), reason="libfa.so not built")
@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump not installed")
def test_each_kernel_in_one_code_object(tmp_path):
    objs = code_objects(tmp_path)
    n = sum(1 for names, _, _ in objs for x in names if x.startswith("_ZN2fa"))
    assert n > 50, f"only {n} kernels found: the disassembly was not parsed"
    dup = kernels_in_several_objects(objs)
    assert not dup, f"{len(dup)} kernels defined in more than one code object, e.g. {dup[:3]}"


def test_build_removes_objects_of_removed_sources(tmp_path):
    """Objects whose source is gone are deleted before linking (a relink that
    picked such objects up once ran an old preprocess kernel)."""
    from io_aware_exact_fa_amd import _build
    for f in ("fa_api.hip.o", "fa_bwd_bf16.hip.o", "fa_fwd.hip.o", "notes.txt"):
        (tmp_path / f).write_text("x")
    srcs = ["/x/csrc/fa_api.hip", "/x/csrc/fa_fwd.hip"]
    assert _build.remove_stale_objects(str(tmp_path), srcs) == ["fa_bwd_bf16.hip.o"]
    assert sorted(p.name for p in tmp_path.iterdir()) == ["fa_api.hip.o", "fa_fwd.hip.o", "notes.txt"]
