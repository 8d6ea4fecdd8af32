"""Build libfp32gemm.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Every source compiles to its own object in parallel, then one shared link.
The matrix-core kernels compile once per line of the instance list
(csrc/fg_mfma_instances.inc) and operand layout: sgemm_mfma_inst.hip with
that line's shape, one translation unit per kernel.
Flags:
  * --offload-arch=gfx950 only;
  * -O3, C++17;
  * the packed-fp32 target feature is disabled for device code (the compiler
    must not form v_pk_* fp32 instructions on its own).
Environment:
  FG_SAVE_TEMPS=1    keep the device assembly (.s) under _build/ for reading
  FG_RESOURCE_USAGE=1  print the per-kernel register/LDS/occupancy remarks (always
                       written to _build/<object>.resources.txt)
  MAX_JOBS           parallel compiles (default: the host's cores, at most 16)

build(instances=..., tuned=..., lib=..., build_dir=...) builds a library from
another instance list (the tile search of autotune.py does).
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
INSTANCES = os.path.join(CSRC, "fg_mfma_instances.inc")
SOURCES = ["fg_api.cpp", "fg_mfma_dispatch.cpp", "sgemm_valu.hip", "sgemm_skinny.hip",
           "fg_elementwise.hip", "fg_probe.hip", "fg_noalloc.hip"]
ENTRY_FIELDS = ("id", "bm", "bn", "waves_m", "waves_n", "bk", "mr", "stages", "dmab", "occ",
                "wps", "fallback")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall"]


def read_instances(path: str = INSTANCES) -> list[dict]:
    """Lines FG_MFMA_ENTRY(...) of an instance list, as dicts (comments
    skipped)."""
    out = []
    for line in open(path):
        line = line.split("//", 1)[0]
        m = re.match(r"\s*FG_MFMA_ENTRY\(([^)]*)\)", line)
        if m:
            vals = [int(v) for v in m.group(1).split(",")]
            if len(vals) != len(ENTRY_FIELDS):
                raise ValueError(f"{path}: bad entry {line.strip()}")
            out.append(dict(zip(ENTRY_FIELDS, vals)))
    return out


def shape_macro(e: dict) -> str:
    return ",".join(str(e[k]) for k in ("bm", "bn", "waves_m", "waves_n", "bk", "mr", "stages",
                                        "dmab", "occ"))


def _compile(src: str, obj: str, extra: list[str], verbose: bool) -> str:
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        if os.environ.get("FG_SAVE_TEMPS"):
            cmd += ["-save-temps=obj"]
        # Per-kernel register / LDS / scratch report of the device pass, kept
        # in <object>.resources.txt (a test checks that no kernel spills to
        # scratch memory; the tile search reads the register counts).
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass warns that it does not know the packed-fp32 feature.
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(obj)}:\n{msgs}")
    remarks = [l for l in msgs.splitlines() if "kernel-resource-usage" in l]
    if src.endswith(".hip"):
        with open(os.path.splitext(obj)[0] + ".resources.txt", "w") as f:
            f.write("\n".join(remarks) + "\n")
    # (the remarks come with source excerpts, "  16 | code" and "  | ^", and
    # with the include chain of the header that holds the kernel)
    others = "\n".join(l for l in msgs.splitlines()
                       if "kernel-resource-usage" not in l and not re.match(r"^\s*\d*\s*\|", l)
                       and not l.startswith("In file included from"))
    if os.environ.get("FG_RESOURCE_USAGE") and msgs.strip():
        print(msgs, flush=True)
    elif others.strip():
        print(others, flush=True)
    return obj


def jobs() -> int:
    n = int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 4)
    return max(1, min(16, n))


def _stale(obj: str, deps: list[str]) -> bool:
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def _deps(src: str, table_files: list[str]) -> list[str]:
    """Files an object depends on: every header of the library; the table
    files (instance list, efficiencies) too unless it is a kernel instance
    (whose shape comes from its -D flags)."""
    heads = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    heads += [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))]
    own = [src] + heads
    return own if src.endswith("sgemm_mfma_inst.hip") else own + table_files


def build(verbose: bool = False, instances: str = INSTANCES, tuned: str | None = None,
          lib: str = LIB, build_dir: str = BUILD, layouts: dict | None = None,
          incremental: bool = False) -> str:
    """Compile every source and every instance of `instances` and link `lib`.
    layouts: {entry id: [(ta, tb), ...]} builds only those operand layouts of
    an entry (the others report hipErrorNotSupported); default all four.
    incremental: keep objects newer than everything they depend on (the tile
    search rebuilds its library after changing only the table)."""
    os.makedirs(build_dir, exist_ok=True)
    defs = [f'-DFG_INSTANCES_INC="{os.path.abspath(instances)}"']
    if tuned:
        defs.append(f'-DFG_TUNED_INC="{os.path.abspath(tuned)}"')
    work = []
    for s in SOURCES:
        work.append((os.path.join(CSRC, s),
                     os.path.join(build_dir, os.path.splitext(s)[0] + ".o"), defs))
    entries = read_instances(instances)
    for e in entries:
        want = set(map(tuple, (layouts or {}).get(e["id"], [(0, 0), (0, 1), (1, 0), (1, 1)])))
        stubs = 0
        for ta in (0, 1):
            for tb in (0, 1):
                if (ta, tb) not in want:
                    stubs |= 1 << (2 * ta + tb)
                    continue
                work.append((os.path.join(CSRC, "sgemm_mfma_inst.hip"),
                             os.path.join(build_dir, f"sgemm_mfma_e{e['id']}_{ta}{tb}.o"),
                             [f"-DFG_ENTRY_ID={e['id']}", f"-DFG_ENTRY_TA={ta}",
                              f"-DFG_ENTRY_TB={tb}", f"-DFG_ENTRY_SHAPE={shape_macro(e)}"]))
        if stubs:
            work.append((os.path.join(CSRC, "sgemm_mfma_inst.hip"),
                         os.path.join(build_dir, f"sgemm_mfma_e{e['id']}_stubs.o"),
                         [f"-DFG_ENTRY_ID={e['id']}", f"-DFG_ENTRY_STUBS={stubs}"]))
    table_files = [os.path.abspath(instances),
                   os.path.abspath(tuned) if tuned else os.path.join(CSRC, "fg_tuned.inc"),
                   os.path.join(CSRC, "fg_model.inc")]
    if incremental:
        keep = [w for w in work if not _stale(w[1], _deps(w[0], table_files))]
        work = [w for w in work if w not in keep]
        kept_objs = [w[1] for w in keep]
    else:
        kept_objs = []
    # The slowest objects first (largest tiles), so the pool drains evenly.
    work.sort(key=lambda w: -int(next((d.split("=")[1].split(",")[0] for d in w[2]
                                       if d.startswith("-DFG_ENTRY_SHAPE=")), "0")))
    if verbose:
        print(f"compiling {len(work)} objects ({len(entries)} matrix-core entries) "
              f"with {jobs()} jobs", flush=True)
    with cf.ThreadPoolExecutor(max_workers=jobs()) as ex:
        objs = list(ex.map(lambda w: _compile(w[0], w[1], w[2], verbose), work)) + kept_objs
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd[:6]) + f" ... ({len(objs)} objects)", flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
