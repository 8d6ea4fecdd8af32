"""Build libfp32gemm.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Each source compiles to its own object in parallel, then one shared link.
Flags:
  * --offload-arch=gfx950 only;
  * -O3, C++17;
  * the packed-fp32 target feature is disabled for device code (the compiler
    must not form v_pk_* fp32 instructions on its own).
Environment:
  FG_SAVE_TEMPS=1    keep the device assembly (.s) under _build/ for reading
  FG_RESOURCE_USAGE=1  print the per-kernel register/LDS/occupancy remarks (always
                       written to _build/<source>.resources.txt)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfp32gemm.so")
SOURCES = ["fg_api.cpp", "sgemm_mfma.hip", "sgemm_valu.hip", "sgemm_skinny.hip",
           "fg_elementwise.hip", "fg_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        if os.environ.get("FG_SAVE_TEMPS"):
            cmd += ["-save-temps=obj"]
        # Per-kernel register / LDS / scratch report of the device pass, kept
        # in _build/<source>.resources.txt (a test checks that no kernel
        # spills to scratch memory).
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass warns that it does not know the packed-fp32 feature.
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    remarks = [l for l in msgs.splitlines() if "kernel-resource-usage" in l]
    if src.endswith(".hip"):
        with open(os.path.join(BUILD, os.path.splitext(src)[0] + ".resources.txt"), "w") as f:
            f.write("\n".join(remarks) + "\n")
    # (the remarks come with source excerpts: "  16 | code" and "  | ^")
    others = "\n".join(l for l in msgs.splitlines()
                       if "kernel-resource-usage" not in l and not re.match(r"^\s*\d*\s*\|", l))
    if verbose or os.environ.get("FG_RESOURCE_USAGE"):
        if msgs.strip():
            print(msgs, flush=True)
    elif others.strip():
        print(others, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
