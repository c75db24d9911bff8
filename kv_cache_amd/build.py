"""Build libdecode_attn.so in-tree for gfx950 (hipcc + g++)."""
from __future__ import annotations

import argparse
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdecode_attn.so")
PROBE_LIB = os.path.join(PKG, "libhbm_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in any kernel of this library.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
             f"-I{CSRC}", f"-I{ROCM}/include"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = True, defines=(), out: str | None = None) -> str:
    """Compile the library (and the probe library) in-tree.  ``defines``
    (e.g. ``["DA_MFMA_QK=0"]``) and ``out`` build a variant of the library at
    another path, for comparisons; the probe library is built only for the
    default output."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    lib = os.path.abspath(out) if out else LIB
    tag = "" if not defines else "_" + hashlib.sha1(" ".join(defines).encode()).hexdigest()[:8]
    plan_o = os.path.join(BUILD_DIR, "plan.o")
    kern_o = os.path.join(BUILD_DIR, f"decode_attn{tag}.o")
    cxx = shutil.which("g++") or "g++"
    dflags = [f"-D{d}" for d in defines]
    _run([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, "plan.cpp"), "-o", plan_o], verbose)
    _run([HIPCC, *HIP_FLAGS, *dflags, "-c", os.path.join(CSRC, "decode_attn.hip"), "-o", kern_o], verbose)
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", plan_o, kern_o, "-o", tmp], verbose)
    os.replace(tmp, lib)
    if out is None:
        tmp = PROBE_LIB + ".tmp"
        _run([HIPCC, *HIP_FLAGS, "-shared", os.path.join(CSRC, "hbm_probe.hip"), "-o", tmp], verbose)
        os.replace(tmp, PROBE_LIB)
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("-q", action="store_true", help="do not echo the commands")
    ap.add_argument("--define", action="append", default=[],
                    help="NAME=VALUE passed to the HIP compile (a library variant)")
    ap.add_argument("--out", default=None, help="output path of a library variant")
    a = ap.parse_args()
    build(verbose=not a.q, defines=a.define, out=a.out)
