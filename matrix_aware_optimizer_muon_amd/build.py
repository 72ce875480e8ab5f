"""Build libmuon.so (HIP for gfx950) in-tree with hipcc.

Every call recompiles every source: this is the "does it build" check as
well as the build.  Objects go to csrc/_build/, the library to lib/.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(CSRC, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmuon.so")
# debug build: every GEMM and elementwise task checks its tile against the
# unit's padded sizes and sets flag bit 2 instead of running out of bounds
DEBUG_LIB = os.path.join(LIBDIR, "libmuon_debug.so")
DEBUG_OBJ = os.path.join(CSRC, "_build_debug")
DEBUG_FLAGS = ["-DMUON_DEBUG_BOUNDS=1"]
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

SOURCES = ["muon_host.cpp", "elementwise.hip", "ns_gemm.hip", "precond.hip", "adamw.hip"]

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-x", "hip",
    # packed fp32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# roctx (named host-side ranges for rocprofv3's marker trace)
ROCM_LIB = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
LINK_FLAGS = [f"-L{ROCM_LIB}", f"-Wl,-rpath,{ROCM_LIB}", "-lrocprofiler-sdk-roctx"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libmuon.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose=False, extra_flags=(), out=None, objdir=None):
    """Compile every source and link the library (default: lib/libmuon.so).
    `extra_flags` and a separate `out`/`objdir` allow variant builds."""
    hipcc = _hipcc()
    obj_dir = objdir or OBJ
    lib = out or LIB
    os.makedirs(obj_dir, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *HIP_FLAGS, *extra_flags, f"-I{INCLUDE}", "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), 4)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = lib + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *LINK_FLAGS, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


def build_debug(verbose=False):
    """The bounds-checking variant, lib/libmuon_debug.so."""
    return build(verbose=verbose, extra_flags=DEBUG_FLAGS, out=DEBUG_LIB, objdir=DEBUG_OBJ)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_debug(verbose="-v" in sys.argv))
