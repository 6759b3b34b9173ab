"""Builds libdmuon_ns.so in-tree for gfx950 with hipcc.

    python -m matrix_optimizer_02_amd.build      (or __graft_entry__.build())

Every HIP source is compiled with packed-fp32 instructions disabled
(-target-feature -packed-fp32-ops); the planner is plain C++ built with g++.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdmuon_ns.so")

HIP_SOURCES = ["api.hip", "k_adamw.hip", "k_diag.hip", "k_elementwise.hip", "k_gemm_bf16.hip", "k_gemm_f32.hip",
               "k_resident.hip", "tune.hip"]
CXX_SOURCES = ["plan.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


HIP_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=fast"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")
    return res


def exported_symbols():
    """Names of the functions include/dmuon_ns.h declares with DMUON_API."""
    import re

    with open(os.path.join(INCLUDE, "dmuon_ns.h")) as f:
        text = f.read()
    return re.findall(r"^DMUON_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)


def build(verbose: bool = False, extra_flags=(), out: str = None, build_dir: str = None) -> str:
    """Compile every source and link libdmuon_ns.so; returns the library path.
    ``extra_flags`` (e.g. -D tuning macros) go to every hipcc compile; ``out``
    and ``build_dir`` redirect the library and the object files."""
    lib = out or LIB
    bdir = build_dir or BUILD
    os.makedirs(bdir, exist_ok=True)
    objs = []
    cc = hipcc()
    for src in HIP_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        _run([cc, *HIP_FLAGS, *extra_flags, f"-I{INCLUDE}", "-c", os.path.join(CSRC, src), "-o", obj],
             verbose)
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden", f"-I{INCLUDE}", "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    version_script = os.path.join(bdir, "exports.map")
    with open(version_script, "w") as f:
        f.write("{ global: " + " ".join(s + ";" for s in exported_symbols()) + " local: *; };\n")
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
          f"-Wl,--version-script={version_script}", "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
