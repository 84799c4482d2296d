"""Build libfa.so (the gfx950 attention library) in-tree with hipcc.

Usage: ``python io_aware_exact_fa_amd/_build.py`` (or ``__graft_entry__.build()``);
run it by path, not as ``-m io_aware_exact_fa_amd._build``, which would import
the package and load the library that is about to be replaced.
Every call compiles from scratch: each ``csrc/*.hip`` file to an object in
``_build/`` (in parallel), then links ``libfa.so.tmp``, checks its device code
(``_devcheck.check_library``: the wait states before every inline-asm
LDS-direct copy, one definition per kernel) and only then installs it as
``libfa.so`` next to this file.  A library that fails the check is deleted and
the build raises, so a register allocation that puts a VALU write of a copy's
SGPR operand too close to the copy never reaches a GPU.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU instructions.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-file flags.  The 16-bit kernels keep their MFMA accumulators in VGPRs
# (the VALU reads S and dP directly, no AGPR copies).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {f"fa_bwd_{t}_d{d}.hip": VGPR_FORM for t in ("bf16", "f16") for d in (64, 128)}
EXTRA["fa_fwd.hip"] = VGPR_FORM
EXTRA["fa_fwd64.hip"] = VGPR_FORM


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(line for line in (r.stderr or "").splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def remove_stale_objects(build_dir: str, sources) -> list:
    """Delete the objects in build_dir whose source is not among `sources`; they
    would define the same template kernels (against older argument layouts) if
    anything linked them.  Returns the names removed."""
    names = {os.path.basename(s) + ".o" for s in sources}
    stale = sorted(f for f in os.listdir(build_dir) if f.endswith(".o") and f not in names)
    for f in stale:
        os.remove(os.path.join(build_dir, f))
    return stale


def _load_devcheck():
    """_devcheck.py, loaded by path (importing the package would load the
    library that is about to be replaced)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_fa_devcheck", os.path.join(PKG, "_devcheck.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def install_checked(tmp: str, lib: str, check) -> dict:
    """Runs `check` on the linked library `tmp`; installs it as `lib` only if
    the check passes, else deletes it and re-raises."""
    try:
        info = check(tmp)
    except Exception:
        os.remove(tmp)
        raise
    os.replace(tmp, lib)
    return info


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    remove_stale_objects(BUILD, sources)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    info = install_checked(tmp, LIB, _load_devcheck().check_library)
    if verbose:
        print(f"built {LIB} (device code checked: {info['lds_dma_loads']} LDS-direct loads, "
              f"{info['kernels']} kernels)")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
