"""Checks of the device code in the built library (no GPU).

The checks themselves live in ``io_aware_exact_fa_amd/_devcheck.py``, which
``build()`` runs on every freshly linked library before installing it (see
that module for the rules: wait states before the inline-asm LDS-direct
copies, one definition per kernel, wait states between a VALU write and an
MFMA reading it).  Here: the scanners flag the hazards they are meant to
flag, the installed library passes the checks, and ``build()`` refuses a
library that fails them."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "io_aware_exact_fa_amd")
LIB = os.path.join(PKG, "libfa.so")


def _by_path(name):
    """A module of the package loaded by path: importing the package would load
    libfa.so, which these CPU checks do not need."""
    spec = importlib.util.spec_from_file_location(f"_fa_{name}", os.path.join(PKG, f"{name}.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


_build = _by_path("_build")
_devcheck = _by_path("_devcheck")
_DMA, OBJDUMP = _devcheck.DMA, _devcheck.OBJDUMP
code_objects, kernels_in_several_objects = _devcheck.code_objects, _devcheck.kernels_in_several_objects
violations = _devcheck.violations
mfma_violations = _devcheck.mfma_violations


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


def test_mfma_scanner_flags_the_hazards():
    """A packed P written by the VALU one wait state before the MFMA that reads
    it as A is flagged, as are B and C operands and the last register of a
    range; two wait states (or a dot product, or an LDS load) are not."""
    mfma = "v_mfma_f32_32x32x16_bf16 a[32:47], v[4:7], v[0:3], a[32:47]"
    assert mfma_violations(["v_cvt_pk_bf16_f32 v4, v13, v15", "s_waitcnt lgkmcnt(0)", mfma])
    assert mfma_violations(["v_cvt_pk_bf16_f32 v7, v13, v15", mfma])
    assert mfma_violations(["v_mov_b32_e32 v2, 0", mfma])
    assert mfma_violations(["v_add_f32_e32 v20, v1, v2",
                            "v_mfma_f32_32x32x16_bf16 v[20:35], v[4:7], v[0:3], v[20:35]"])
    assert not mfma_violations(["v_cvt_pk_bf16_f32 v4, v13, v15", "s_nop 1", mfma])
    assert not mfma_violations(["v_cvt_pk_bf16_f32 v4, v13, v15", "v_add_f32_e32 v9, v1, v2",
                                "v_mul_f32_e32 v10, v1, v2", mfma])
    assert not mfma_violations(["v_dot2c_f32_bf16_e32 v4, v1, v2", mfma])
    assert not mfma_violations(["ds_read_b64_tr_b16 v[0:1], v29 offset:4096", mfma])
    assert not mfma_violations(["v_cvt_pk_bf16_f32 v8, v13, v15", mfma])       # another VGPR
    assert mfma_violations(["s_nop 1", "s_nop 0", mfma], targets={1})        # reached by a branch


@pytest.mark.skipif(not os.path.exists(LIB), reason="libfa.so not built")
@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump not installed")
def test_every_mfma_has_its_wait_states(tmp_path):
    objs = code_objects(LIB, str(tmp_path))
    n = sum(1 for _, lines, _ in objs for ins in lines if ins and _devcheck.MFMA.match(ins))
    assert n > 1000, f"only {n} MFMAs found: the disassembly was not parsed"
    bad = [v for _, lines, targets in objs for v in mfma_violations(lines, targets)]
    assert not bad, f"{len(bad)} of {n} MFMAs too soon after a VALU write, e.g. " + \
        "; ".join(f"{p!r} {w} wait states before {ins!r}" for _, ins, p, w in bad[:4])


@pytest.mark.skipif(not os.path.exists(LIB), reason="libfa.so not built")
@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump not installed")
def test_every_lds_dma_load_has_its_wait_states(tmp_path):
    objs = code_objects(LIB, str(tmp_path))
    n = sum(1 for _, lines, _ in objs for ins in lines if ins and _DMA.match(ins))
    assert n > 1000, f"only {n} LDS-direct loads found: the disassembly was not parsed"
    assert sum(len(t) for _, _, t in objs) > 100, "no branch targets found"
    bad = [v for _, lines, targets in objs for v in violations(lines, targets)]
    assert not bad, f"{len(bad)} of {n} LDS-direct loads too soon after an SGPR/M0 write, e.g. " + \
        "; ".join(f"{p!r} {w} wait states before {ins!r}" for _, ins, p, w in bad[:4])


@pytest.mark.skipif(not os.path.exists(LIB), reason="libfa.so not built")
@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump not installed")
def test_each_kernel_in_one_code_object(tmp_path):
    objs = code_objects(LIB, str(tmp_path))
    n = sum(1 for names, _, _ in objs for x in names if x.startswith("_ZN2fa"))
    assert n > 50, f"only {n} kernels found: the disassembly was not parsed"
    dup = kernels_in_several_objects(objs)
    assert not dup, f"{len(dup)} kernels defined in more than one code object, e.g. {dup[:3]}"


def test_build_removes_objects_of_removed_sources(tmp_path):
    """Objects whose source is gone are deleted before linking (a relink that
    picked such objects up once ran an old preprocess kernel)."""
    for f in ("fa_api.hip.o", "fa_bwd_bf16.hip.o", "fa_fwd.hip.o", "notes.txt"):
        (tmp_path / f).write_text("x")
    srcs = ["/x/csrc/fa_api.hip", "/x/csrc/fa_fwd.hip"]
    assert _build.remove_stale_objects(str(tmp_path), srcs) == ["fa_bwd_bf16.hip.o"]
    assert sorted(p.name for p in tmp_path.iterdir()) == ["fa_api.hip.o", "fa_fwd.hip.o", "notes.txt"]


def test_build_installs_only_a_checked_library(tmp_path):
    """build() links to a temporary file and installs it only after the device
    code check passed; a failing check deletes it and leaves the installed
    library alone."""
    lib, tmp = tmp_path / "libfa.so", tmp_path / "libfa.so.tmp"
    lib.write_text("old")
    tmp.write_text("new")

    def bad(path):
        raise RuntimeError("device-code check: 1 of 4440 LDS-direct loads too soon")

    with pytest.raises(RuntimeError, match="too soon"):
        _build.install_checked(str(tmp), str(lib), bad)
    assert not tmp.exists() and lib.read_text() == "old"
    tmp.write_text("new")
    assert _build.install_checked(str(tmp), str(lib), lambda p: {"ok": p}) == {"ok": str(tmp)}
    assert not tmp.exists() and lib.read_text() == "new"


def test_build_runs_the_device_code_check():
    """build() passes the linked library through _devcheck.check_library (the
    guard against the copy hazard that once faulted), not only the tests."""
    import inspect
    src = inspect.getsource(_build.build)
    assert "install_checked(" in src and "check_library" in src
    assert "os.replace" not in src   # the only install path is install_checked
