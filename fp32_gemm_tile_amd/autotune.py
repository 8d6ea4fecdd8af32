"""Offline tuner for the tile-configuration table: a search over kernel
instances, and the fit of the cost model that picks among the kept ones.

The library picks a table entry per call with a cost model (fg_api.cpp) that
holds, for every matrix-core entry, two efficiencies: ``eff`` (fraction of
the fp32 matrix peak a wave reaches with its SIMD full) and ``eff1`` (the same
with one wave per SIMD); the few-row entry has one, dividing its modelled
time per step of K.

Tile search (the empirical configuration search of "How to get a matmul
kernel into the top percentile (worklog)", section "Extra": a configuration
found for one GPU is retuned for another, there by changing the k-tile
depth; and "Matmul II: register blocking, warp tiling, tensor cores",
section 8: a library carries a family of tile variants found by search and
chooses among them per shape):

  1. ``--build-search`` (any host): enumerate the kernel instances the
     template accepts within the machine's limits -- workgroup tile
     BM x BN in {64, 128, 256}^2, wave grid, k-tile depth BK in {8, 16, 32},
     MFMA block 32x32x2 or 16x16x4, a 3- or 4-deep direct-to-LDS ring with
     16- or 4-byte loads, occupancy -- write them as an instance list next to
     this module (``_search/``) and build a search library from it.
  2. ``--search REPORT`` (on the GPU): load that library, check every
     instance on integer-valued inputs (bit-exact), time it on the tuning
     shapes, fit its two efficiencies, write REPORT (JSON); then
     ``--refine REPORT`` re-times the instances near the fastest of each
     shape in interleaved rounds.
  3. ``--select REPORT`` (any host): keep a small set of instances that
     covers every tuning shape within 1% of the fastest instance found for
     it, plus the 4-byte-load entries unaligned rows need, and write
     ``csrc/fg_mfma_instances.inc`` (the table's matrix-core rows) and
     ``csrc/fg_tuned.inc`` (their efficiencies). Rebuild the library after.

Refit only (no search): ``python -m fp32_gemm_tile_amd.autotune [--quick]
[--write] [--report PATH]`` times every entry of the built library on the
tuning shapes, refits the efficiencies and checks that the model's picks
agree with the measured best; ``--from-report PATH --write`` regenerates
``csrc/fg_tuned.inc`` from a saved report on any host.
"""
from __future__ import annotations

import argparse
import datetime
import json
import math
import os
import re
import sys
import time

import fp32_gemm_tile_amd as fg

HERE = os.path.dirname(os.path.abspath(__file__))
INC_PATH = os.path.join(HERE, "csrc", "fg_tuned.inc")

# (M, N, K, transA, transB, lda, ldb, ldc); None = dense leading dimension.
SHAPES = [
    (s, s, s, "N", "N", None, None, None) for s in (256, 512, 768, 1024, 1536, 2048, 3072,
                                                    4096, 6144, 8192)
] + [
    (1024, 8192, 8192, "N", "N", None, None, None),
    (2048, 8192, 8192, "N", "N", None, None, None),
    (8192, 1024, 8192, "N", "N", None, None, None),
    (4096, 4096, 1024, "N", "N", None, None, None),
    (8192, 8192, 512, "N", "N", None, None, None),
    (16384, 16384, 256, "N", "N", None, None, None),
    (4096, 4096, 4096, "N", "T", None, None, None),
    (4096, 4096, 4096, "T", "N", None, None, None),
    (128, 4096, 4096, "N", "N", None, None, None),
    (256, 4096, 4096, "N", "N", None, None, None),
    (512, 8192, 8192, "N", "N", None, None, None),
    (3001, 2047, 1025, "T", "N", 3001, 2047, 2047),
    (2049, 2049, 2049, "N", "N", None, None, None),
]
QUICK = [SHAPES[i] for i in (3, 5, 7, 9, 10, 15, 18, 21, 22)]


def _lds(shape):
    M, N, K, ta, tb, lda, ldb, ldc = shape
    lda = lda or (M if ta == "T" else K)
    ldb = ldb or (K if tb == "T" else N)
    ldc = ldc or N
    return lda, ldb, ldc


def _aligned(shape):
    lda, ldb, _ = _lds(shape)
    return lda % 4 == 0 and ldb % 4 == 0


def candidates(shape):
    """Table entries worth timing on a shape: matrix-core entries (those
    with 16-byte direct-to-LDS loads only on 16-byte aligned rows, where
    they run themselves rather than their fallback) and the few-row entry on
    shapes of at most 512 rows (its model is fitted on those of at most 256,
    where it can win)."""
    M = shape[0]
    out = []
    for i in range(fg.fg_num_configs()):
        c = fg.fg_get_config(i)
        if c["kind"] == fg.FG_KIND_SKINNY and M <= 512:
            out.append(i)
        elif c["kind"] == fg.FG_KIND_MFMA:
            if not _aligned(shape) and c["stages"] >= 3 and "_dw" not in c["name"]:
                continue   # 16-byte direct-to-LDS loads need 16-byte aligned rows
            out.append(i)
    return out


def time_entries(shape, entries, budget_s=0.05):
    """Mean seconds per call of each entry (back-to-back calls between one
    event pair, after two warm-up calls)."""
    import torch
    M, N, K, ta, tb = shape[:5]
    lda, ldb, ldc = _lds(shape)
    a_rows, b_rows = (K if ta == "T" else M), (N if tb == "T" else K)
    g = torch.Generator(device="cuda").manual_seed(M * 31 + N * 7 + K)
    A = torch.rand(a_rows * lda, device="cuda", generator=g) * 2 - 1
    B = torch.rand(b_rows * ldb, device="cuda", generator=g) * 2 - 1
    C = torch.empty(M * ldc, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    out = {}
    for e in entries:
        def call():
            st = fg.fg_sgemm_ex(ta, tb, M, N, K, 1.0, A.data_ptr(), lda, B.data_ptr(), ldb, 0.0,
                                C.data_ptr(), ldc, sp, e)
            if st != fg.FG_OK:
                raise fg.FgError(st, fg.fg_last_bad_arg(), fg.fg_last_error())
        call()
        call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        call()
        torch.cuda.synchronize()
        once = max(time.perf_counter() - t0, 1e-6)
        reps = int(min(20, max(3, budget_s / once)))
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            call()
        ev1.record(stream)
        torch.cuda.synchronize()
        out[e] = ev0.elapsed_time(ev1) * 1e-3 / reps
    return out


def fit_entry(entry, samples, wps_gt_1, step=0.01):
    """Efficiencies of one modelled entry that minimise the squared log
    error of the model against `samples` = [(M, N, K, seconds), ...]: a grid
    search over eff in [0.30, 1.00] and, when several waves can share a SIMD,
    eff1 in [0.20, eff] (steps of `step`). Leaves the library holding the
    best pair; returns (eff, eff1, rms log error)."""
    best = None
    effs = [round(0.30 + step * i, 2) for i in range(int(round(0.70 / step)) + 1)]
    for eff in effs:
        ones = [round(0.20 + step * i, 2) for i in range(int(round((eff - 0.20) / step)) + 1)] \
            if wps_gt_1 else [eff]
        for eff1 in ones:
            fg.fg_set_efficiency(entry, eff, eff1)
            err = 0.0
            for M, N, K, t in samples:
                err += math.log(fg.fg_estimate_seconds(M, N, K, entry) / t) ** 2
            if best is None or err < best[2]:
                best = (eff, eff1, err)
    eff, eff1, err = best
    fg.fg_set_efficiency(entry, eff, eff1)
    return eff, eff1, math.sqrt(err / max(1, len(samples)))


def eff1_matters(entry):
    """Whether the model of an entry ever uses its one-wave efficiency (only
    when several of its waves can share a SIMD)."""
    old = fg.fg_get_efficiency(entry)
    probe = [(256, 256, 256), (1024, 1024, 1024), (128, 4096, 4096), (4096, 4096, 4096)]
    try:
        fg.fg_set_efficiency(entry, old[0], 0.25)
        a = [fg.fg_estimate_seconds(M, N, K, entry) for M, N, K in probe]
        fg.fg_set_efficiency(entry, old[0], 0.75)
        b = [fg.fg_estimate_seconds(M, N, K, entry) for M, N, K in probe]
    finally:
        fg.fg_set_efficiency(entry, *old)
    return a != b


def write_inc(fitted, n_shapes, path=INC_PATH):
    lines = ["// Cost-model efficiencies of the modelled table entries: {id, eff, eff1}.",
             "// eff: fraction of the fp32 matrix peak a wave reaches with its SIMD full;",
             "// eff1: the same with one wave per SIMD (the few-row entry: eff divides",
             "// its modelled step time, eff1 unused). Written by",
             "// fp32_gemm_tile_amd/autotune.py (--write) from timings of every entry on",
             f"// {n_shapes} shapes on one MI355X, {datetime.date.today().isoformat()}."]
    for e in sorted(fitted):
        eff, eff1, _ = fitted[e]
        name = fg.fg_get_config(e)["name"]
        key = "FG_ID_SKINNY" if name == SKINNY else e
        lines.append(f"{{{key}, {eff:.3f}, {eff1:.3f}}},  // {name}")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


# ---------------------------------------------------------------------------
# Tile search

ROOT = os.path.dirname(HERE)
INSTANCES_PATH = os.path.join(HERE, "csrc", "fg_mfma_instances.inc")
SEARCH_DIR = os.path.join(HERE, "_search")
SEARCH_INC = os.path.join(SEARCH_DIR, "fg_mfma_instances.inc")
SEARCH_TUNED = os.path.join(SEARCH_DIR, "fg_tuned.inc")
SEARCH_LIB = os.path.join(SEARCH_DIR, "libfp32gemm_search.so")
SEARCH_BUILD = os.path.join(ROOT, "_build", "search")
FIXED_NAMES = ("valu_128x128x8_t8x8", "valu_64x64x8_t4x4", "few_rows")  # after the
# matrix-core rows, in this order (fg_api.cpp lists them itself)
SKINNY = "few_rows"
SKINNY_OLD = "valu_skinny_m8"   # its name in reports written before it had a matrix-core kernel


def fixed_ids():
    """{name: table id} of the vector-ALU and few-row rows of the loaded library."""
    return {c["name"]: c["id"] for c in fg.configs() if c["kind"] != fg.FG_KIND_MFMA}


def _skinny_id(report):
    ids = report.get("fixed_ids", {})
    return ids.get(SKINNY, ids.get(SKINNY_OLD))
LDS_BYTES = 160 * 1024
SHAPE_KEYS = ("bm", "bn", "waves_m", "waves_n", "bk", "mr", "stages", "dmab", "occ")

# Workgroup tile and wave grid (BM, BN, WAVES_M, WAVES_N, MR) of the search:
# square-ish wave tiles (a wave's LDS reads grow with the tile's perimeter,
# its MFMAs with the area: "Matmul II", section 5) from 32 x 32 to 128 x 128
# with 32 x 32 blocks, and 32 x 32 to 64 x 64 with 16 x 16 blocks.
TILES = [
    (64, 64, 2, 2, 32), (64, 64, 2, 2, 16),
    (128, 64, 2, 2, 32), (128, 64, 2, 2, 16), (64, 128, 2, 2, 32), (64, 128, 2, 2, 16),
    (128, 128, 2, 2, 32), (128, 128, 2, 2, 16), (128, 128, 4, 2, 32), (128, 128, 2, 4, 32),
    (256, 128, 2, 2, 32), (128, 256, 2, 2, 32), (256, 128, 4, 2, 32), (128, 256, 2, 4, 32),
    (256, 128, 2, 1, 32), (256, 256, 2, 2, 32), (256, 256, 4, 2, 32), (256, 256, 2, 4, 32),
]

# Shapes the search times (the refit shapes plus rows that are not 16-byte
# aligned, which only the 4-byte-load and register-staged entries can take,
# and the NT headline).
SEARCH_SHAPES = SHAPES + [
    (8192, 8192, 8192, "N", "T", None, None, None),
    (1025, 1025, 1025, "N", "N", None, None, None),
    (4095, 4095, 4095, "N", "N", None, None, None),
    (6001, 4001, 2001, "T", "N", None, None, None),
]


def needs_aligned_rows(e):
    """16-byte direct-to-LDS loads: rows of A and B must start 16-byte aligned."""
    return e["stages"] >= 3 and e["dmab"] == 16


def registers(e):
    """(accumulator, operand-fragment) registers per lane of an instance."""
    wm, wn = e["bm"] // e["waves_m"], e["bn"] // e["waves_n"]
    mb, nb = wm // e["mr"], wn // e["mr"]
    kpl = e["bk"] // (64 // e["mr"])
    return mb * nb * e["mr"] * e["mr"] // 64, 2 * kpl * (mb + nb)


def valid_instance(e):
    """The template's own constraints (sgemm_mfma.h) and the machine's."""
    nw = e["waves_m"] * e["waves_n"]
    wm, wn = e["bm"] // e["waves_m"], e["bn"] // e["waves_n"]
    if wm % e["mr"] or wn % e["mr"] or wm // e["mr"] not in (1, 2, 4) or \
            wn // e["mr"] not in (1, 2, 4):
        return False
    kpl = e["bk"] // (64 // e["mr"])
    if not (kpl == 2 or kpl % 4 == 0):
        return False
    if e["stages"] * (e["bm"] + e["bn"]) * e["bk"] * 4 > LDS_BYTES:
        return False
    if e["stages"] >= 3:
        w = e["dmab"] // 4
        per = [(bx * e["bk"]) // (64 * w) for bx in (e["bm"], e["bn"])]
        if any((bx * e["bk"]) % (64 * w * nw) for bx in (e["bm"], e["bn"])):
            return False
        if (e["stages"] - 3) * sum(p // nw for p in per) >= 64:
            return False
    acc, frag = registers(e)
    return acc <= 256 and acc + frag + 48 <= 512


def search_space():
    """Instances the search times: every TILES shape with BK in {8, 16, 32}
    and 16-byte direct-to-LDS loads, plus the 4-byte form for tiles of at
    most 128 x 128; the ring as deep as the LDS allows (at most 4) for the
    occupancy the registers allow (two waves per SIMD when a wave needs at
    most half of a lane's 512 registers)."""
    out = []
    for bm, bn, wm_, wn_, mr in TILES:
        nw = wm_ * wn_
        for bk in (8, 16, 32):
            for dmab in (16, 4):
                if dmab == 4 and bm * bn > 128 * 128:
                    continue
                e = dict(bm=bm, bn=bn, waves_m=wm_, waves_n=wn_, bk=bk, mr=mr, dmab=dmab)
                acc, frag = registers(e)
                occ = 2 if acc + frag + 56 <= 256 else 1
                wgs = max(1, occ * 4 // nw)   # workgroups per CU at that occupancy
                for st in (4, 3):
                    if st * (bm + bn) * bk * 4 * wgs <= LDS_BYTES:
                        break
                else:
                    occ, st = 1, (4 if 4 * (bm + bn) * bk * 4 <= LDS_BYTES else 3)
                e.update(stages=st, occ=occ)
                if valid_instance(e):
                    out.append(e)
    return out


def shape_key(e):
    return tuple(int(e[k]) for k in SHAPE_KEYS)


def instance_name(e):
    """The table's name of an instance (as fg_api.cpp builds it)."""
    n = f"mfma_{e['bm']}x{e['bn']}x{e['bk']}_w{e['waves_m']}x{e['waves_n']}"
    if e["stages"] > 2:
        n += f"_s{e['stages']}"
        if e["dmab"] == 4:
            n += "_dw"
    if e["mr"] == 16:
        n += "_m16"
    return n


INSTANCE_DOC = """\
//
// FG_MFMA_ENTRY(id, BM, BN, WAVES_M, WAVES_N, BK, MR, STAGES, DMAB, OCC, WPS, FALLBACK)
//   id        table index (fg_get_config): 0 .. n-1 in this order; the
//             vector-ALU and few-row rows of fg_api.cpp follow them
//   BM x BN   workgroup tile; WAVES_M x WAVES_N wavefronts of
//             (BM / WAVES_M) x (BN / WAVES_N)
//   BK        k-tile depth; MR 32 (v_mfma_f32_32x32x2_f32) or 16
//             (v_mfma_f32_16x16x4_f32) blocks
//   STAGES    2: register-staged LDS double buffer; 3 or 4: direct-to-LDS ring
//   DMAB      bytes per lane of one direct-to-LDS load (16: rows of A and B
//             must start 16-byte aligned; 4: any rows)
//   OCC       waves per SIMD the register allocation must allow
//   WPS       waves of this kernel one SIMD holds at once (the compiler's
//             occupancy for its registers, capped by the LDS it needs)
//   FALLBACK  entry run instead when a row of A or B is not 16-byte aligned
//             (-1: any alignment is fine)"""


def write_instance_list(path, entries, title):
    from fp32_gemm_tile_amd.build import ENTRY_FIELDS
    lines = [f"// {line}" for line in title.splitlines()] + INSTANCE_DOC.splitlines()
    for e in sorted(entries, key=lambda e: e["id"]):
        vals = ", ".join(str(int(e[k])) for k in ENTRY_FIELDS)
        lines.append(f"FG_MFMA_ENTRY({vals})  // {instance_name(e)}")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def occupancy(build_dir, e):
    """Waves of an instance one SIMD holds: the compiler's occupancy report
    (registers) over the built layouts, capped by the LDS its workgroups
    need."""
    import glob
    import re
    occ = []
    for path in glob.glob(os.path.join(build_dir, f"sgemm_mfma_e{e['id']}_[01][01].resources.txt")):
        occ += [int(v) for v in re.findall(r"Occupancy \[waves/SIMD\]: (\d+)", open(path).read())]
    if not occ:
        raise RuntimeError(f"no resource report for entry {e['id']} in {build_dir}")
    nw = e["waves_m"] * e["waves_n"]
    lds = e["stages"] * (e["bm"] + e["bn"]) * e["bk"] * 4
    by_lds = max(1, (LDS_BYTES // lds) * nw // 4)
    return max(1, min(min(occ), by_lds))


def spills(build_dir, e):
    import glob
    import re
    out = 0
    for path in glob.glob(os.path.join(build_dir, f"sgemm_mfma_e{e['id']}_*.resources.txt")):
        out = max([out] + [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)",
                                                       open(path).read())])
    return out


def search_layouts(e):
    """Operand layouts the search times an instance in: those of the search
    shapes it can take."""
    out = set()
    for sh in SEARCH_SHAPES:
        if needs_aligned_rows(e) and not _aligned(sh):
            continue
        out.add((int(sh[3] == "T"), int(sh[4] == "T")))
    return sorted(out)


def build_search(verbose=False):
    """Write the search instance list (the table's current entries at their
    ids, then the search space) and build the search library; the waves per
    SIMD of every instance come from the compiler's report of that build."""
    from fp32_gemm_tile_amd import build as fgbuild
    current = fgbuild.read_instances(INSTANCES_PATH)
    # one instance per shape whatever its occupancy bound (names stay unique)
    seen = {shape_key(e)[:-1] for e in current}
    entries = [dict(e) for e in current]
    nid = len(entries)
    assert sorted(e["id"] for e in entries) == list(range(nid)), "table ids are not 0 .. n-1"
    generic = next(e["id"] for e in current if not needs_aligned_rows(e))
    for e in search_space():
        if shape_key(e)[:-1] in seen:
            continue
        seen.add(shape_key(e)[:-1])
        entries.append(dict(e, id=nid, wps=1, fallback=generic if needs_aligned_rows(e) else -1))
        nid += 1
    layouts = {e["id"]: search_layouts(e) for e in entries}
    os.makedirs(SEARCH_DIR, exist_ok=True)
    with open(SEARCH_TUNED, "w") as f:
        f.write("// (search library: default efficiencies)\n")
    write_instance_list(SEARCH_INC, entries, "Tile-search instances (autotune.py --build-search)")
    print(f"[search] {len(entries)} instances, "
          f"{sum(len(v) for v in layouts.values())} kernels", flush=True)
    fgbuild.build(verbose, instances=SEARCH_INC, tuned=SEARCH_TUNED, lib=SEARCH_LIB,
                  build_dir=SEARCH_BUILD, layouts=layouts, incremental=True)
    for e in entries:
        e["wps"] = occupancy(SEARCH_BUILD, e)
        e["spill"] = spills(SEARCH_BUILD, e)
    write_instance_list(SEARCH_INC, entries, "Tile-search instances (autotune.py --build-search)")
    fgbuild.build(verbose, instances=SEARCH_INC, tuned=SEARCH_TUNED, lib=SEARCH_LIB,
                  build_dir=SEARCH_BUILD, layouts=layouts, incremental=True)
    with open(os.path.join(SEARCH_DIR, "instances.json"), "w") as f:
        json.dump(entries, f, indent=0)
    return entries


def check_instance_exact(e, lib_entry):
    """Integer-valued inputs (every partial sum exact in binary32) on ragged
    shapes with padded, 16-byte aligned rows, in each layout the instance was
    built for: the result must equal the exact product bit for bit."""
    import numpy as np
    import torch
    for ta, tb in search_layouts(e):
        for (M, N, K, alpha, beta) in [(200, 136, 72, 1.0, 0.0), (97, 131, 45, -1.0, 2.0),
                                      (300, 260, 1030, 0.5, -1.0)]:
            rng = np.random.default_rng(M + N + K + e["id"])
            pad = lambda n: (n + 3) // 4 * 4
            a_rows, a_cols = (K, M) if ta else (M, K)
            b_rows, b_cols = (N, K) if tb else (K, N)
            lda, ldb, ldc = pad(a_cols), pad(b_cols), pad(N)
            A = rng.integers(-8, 9, (a_rows, lda)).astype(np.float32)
            B = rng.integers(-8, 9, (b_rows, ldb)).astype(np.float32)
            C = rng.integers(-8, 9, (M, ldc)).astype(np.float32)
            opA = (A[:, :a_cols].T if ta else A[:, :a_cols]).astype(np.int64)
            opB = (B[:, :b_cols].T if tb else B[:, :b_cols]).astype(np.int64)
            want = (alpha * (opA @ opB) + beta * C[:, :N]).astype(np.float32)
            dA, dB, dC = (torch.from_numpy(x).cuda() for x in (A, B, C))
            st = fg.fg_sgemm_ex(ta, tb, M, N, K, alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb,
                                beta, dC.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream,
                                lib_entry)
            if st != fg.FG_OK:
                return f"status {st}: {fg.fg_last_error()}"
            got = dC.cpu().numpy()[:, :N]
            if not np.array_equal(got, want):
                bad = np.argwhere(got != want)
                return f"{'NT'[ta]}{'NT'[tb]} {M}x{N}x{K}: {len(bad)} wrong, first {bad[0].tolist()}"
    return None


def run_search(report_path, shapes=None):
    """On the GPU: check, time and fit every instance of the search library."""
    import torch
    fg.load_library(SEARCH_LIB)
    entries = json.load(open(os.path.join(SEARCH_DIR, "instances.json")))
    shapes = shapes or SEARCH_SHAPES
    report = {"date": datetime.datetime.now().isoformat(timespec="seconds"),
              "device": torch.cuda.get_device_name(0), "fixed_ids": fixed_ids(),
              "instances": [], "shapes": []}
    skinny = _skinny_id(report)
    ok_ids = []
    for n, e in enumerate(entries):
        if n % 10 == 0:
            print(f"[search] checking instance {n} of {len(entries)}", flush=True)
        err = check_instance_exact(e, e["id"]) if not e.get("spill") else "spills"
        rec = dict(e, name=instance_name(e), exact=err is None, error=err)
        report["instances"].append(rec)
        if err is None:
            ok_ids.append(e["id"])
        else:
            print(f"[search] {instance_name(e)} rejected: {err}", flush=True)
    print(f"[search] {len(ok_ids)} of {len(entries)} instances exact", flush=True)
    by_id = {e["id"]: e for e in entries}
    timings = []
    for sh in shapes:
        ta, tb = int(sh[3] == "T"), int(sh[4] == "T")
        cand = [i for i in ok_ids if (ta, tb) in map(tuple, search_layouts(by_id[i]))
                and (_aligned(sh) or not needs_aligned_rows(by_id[i]))]
        if sh[0] <= 512:
            cand.append(skinny)   # the few-row entry, for reference
        # bring the clock up before the first candidate of a shape
        time_entries(sh, cand[:1], budget_s=0.2)
        t = time_entries(sh, cand)
        timings.append((sh, t))
        best = min(t, key=t.get)
        report["shapes"].append({"shape": list(sh), "seconds": {str(k): v for k, v in t.items()}})
        print(f"[search] {sh[:5]}: {len(cand)} timed, best {fg.fg_get_config(best)['name']} "
              f"{2 * sh[0] * sh[1] * sh[2] / t[best] / 1e12:.1f} TFLOP/s", flush=True)
        with open(report_path, "w") as f:
            json.dump(report, f)
    for n, rec in enumerate(report["instances"]):
        if n % 10 == 0:
            print(f"[search] fitting instance {n} of {len(report['instances'])}", flush=True)
        if not rec["exact"]:
            continue
        samples = [(sh[0], sh[1], sh[2], t[rec["id"]]) for sh, t in timings if rec["id"] in t]
        if samples:
            eff, eff1, rms = fit_entry(rec["id"], samples, eff1_matters(rec["id"]))
            rec.update(eff=eff, eff1=eff1, rms_log_error=rms)
    with open(report_path, "w") as f:
        json.dump(report, f)
    print(f"[search] report written to {report_path}", flush=True)
    return report


def refine_search(report_path, window=1.06, rounds=3, budget_s=0.25):
    """On the GPU: re-time, on every shape of a search report, the instances
    within `window` of its fastest, in `rounds` interleaved rounds with a
    longer budget each; the report keeps the fastest round of each as
    "refined" seconds (the selection uses them). Short kernels need this: one
    quick pass puts instances within a few percent in a random order."""
    import torch  # noqa: F401
    fg.load_library(SEARCH_LIB)
    report = json.load(open(report_path))
    for rec in report["shapes"]:
        sh = tuple(rec["shape"])
        t = {int(k): v for k, v in rec["seconds"].items()}
        best = min(t.values())
        cand = sorted(k for k, v in t.items() if v <= window * best)
        time_entries(sh, cand[:1], budget_s=0.2)   # clock up
        runs = [time_entries(sh, cand, budget_s) for _ in range(rounds)]
        rec["refined"] = {str(k): min(r[k] for r in runs) for k in cand}
        b = min(rec["refined"], key=rec["refined"].get)
        print(f"[refine] {sh[:5]}: {len(cand)} re-timed, best "
              f"{fg.fg_get_config(int(b))['name']} "
              f"{2 * sh[0] * sh[1] * sh[2] / rec['refined'][b] / 1e12:.1f} TFLOP/s", flush=True)
        with open(report_path, "w") as f:
            json.dump(report, f)
    return report


# Few-row shapes the few-row entry's efficiency is also fitted on (the tile
# search's shapes start at 128 rows): the decode shapes of every layout of B,
# 16 to 64 rows, and N = K = 4096.
FEW_SHAPES = [(M, N, N, "N", tb, None, None, None) for M, N, tb in
              [(1, 8192, "N"), (1, 8192, "T"), (4, 8192, "T"), (8, 8192, "N"), (8, 8192, "T"),
               (16, 8192, "N"), (32, 8192, "N"), (32, 8192, "T"), (64, 8192, "N"),
               (8, 4096, "N"), (32, 4096, "N"), (64, 4096, "N")]]


def retime_few_rows(report_path, rounds=3, budget_s=0.25, write=True):
    """On the GPU: the few-row entry's kernels change apart from the tile
    search, so re-time that entry of the built library on every search shape
    with at most 512 rows (best of `rounds` passes), put the times in the
    report in place of the few-row times it holds, refit the entry's
    efficiency from them and from FEW_SHAPES, and rewrite its row of
    fg_tuned.inc."""
    import torch  # noqa: F401
    fg.load_library()
    report = json.load(open(report_path))
    sk_rep = _skinny_id(report)
    sk = [c["id"] for c in fg.configs() if c["kind"] == fg.FG_KIND_SKINNY][0]
    samples = []
    for rec in report["shapes"]:
        sh = tuple(rec["shape"])
        if sh[0] > 512:
            continue
        time_entries(sh, [sk], budget_s=0.2)   # clock up
        t = min(time_entries(sh, [sk], budget_s)[sk] for _ in range(rounds))
        rec["seconds"][str(sk_rep)] = t
        rec.setdefault("refined", {})[str(sk_rep)] = t
        samples.append((sh[0], sh[1], sh[2], t))
        print(f"[few-rows] {sh[:5]}: {t * 1e6:.1f} us, "
              f"{2 * sh[0] * sh[1] * sh[2] / t / 1e12:.1f} TFLOP/s", flush=True)
    few = []
    for sh in FEW_SHAPES:
        time_entries(sh, [sk], budget_s=0.2)
        t = min(time_entries(sh, [sk], budget_s)[sk] for _ in range(rounds))
        samples.append((sh[0], sh[1], sh[2], t))
        few.append({"shape": list(sh[:5]), "seconds": t})
        print(f"[few-rows] {sh[:5]}: {t * 1e6:.1f} us, "
              f"{4 * sh[1] * sh[2] / t / 1e9:.0f} GB/s of op(B)", flush=True)
    eff, eff1, rms = fit_entry(sk, samples, False)
    report["few_rows"] = {"date": datetime.datetime.now().isoformat(timespec="seconds"),
                          "eff": eff, "eff1": eff1, "rms_log_error": rms,
                          "shapes": len(samples), "few_row_shapes": few}
    print(f"[few-rows] fitted eff {eff:.2f}, rms log error {rms:.3f}", flush=True)
    if write:
        with open(report_path, "w") as f:
            json.dump(report, f)
        lines = open(INC_PATH).read().splitlines()
        lines = [f"{{FG_ID_SKINNY, {eff:.3f}, {eff1:.3f}}},  // {SKINNY}"
                 if l.startswith("{FG_ID_SKINNY,") else l for l in lines]
        with open(INC_PATH, "w") as f:
            f.write("\n".join(lines) + "\n")
    return report


MODEL_INC = os.path.join(HERE, "csrc", "fg_model.inc")
# Constants of the cost model the search's timings can fix (the split-K slice
# rate has no timing in them and keeps its default), with the factors tried
# around the current value in each sweep.
FIT_CONSTANTS = ("launch", "store_bw", "store_exposed", "stream_bw", "few_fixed", "few_mfma")
FIT_FACTORS = (0.5, 0.7, 0.85, 0.93, 1.0, 1.07, 1.18, 1.4, 2.0)


def model_samples(report):
    """{table entry id: [(M, N, K, seconds)]} of the built library's
    modelled entries from a search report: each matrix-core entry's instance
    times (matched by shape), and the few-row entry's times on the search
    shapes and on FEW_SHAPES (written by retime_few_rows)."""
    from fp32_gemm_tile_amd import build as fgbuild
    by_key = {shape_key(r): r["id"] for r in report["instances"]}
    out = {}
    for e in fgbuild.read_instances(INSTANCES_PATH):
        rid = by_key.get(shape_key(e))
        out[e["id"]] = [(sh[0], sh[1], sh[2], t[rid]) for sh, t in _report_times(report)
                        if rid in t]
    sk = [c["id"] for c in fg.configs() if c["kind"] == fg.FG_KIND_SKINNY][0]
    sk_rep = _skinny_id(report)
    few = [(sh[0], sh[1], sh[2], t[sk_rep]) for sh, t in _report_times(report)
           if sh[0] <= 512 and sk_rep in t]
    few += [(r["shape"][0], r["shape"][1], r["shape"][2], r["seconds"])
            for r in report.get("few_rows", {}).get("few_row_shapes", [])]
    out[sk] = few
    return out


def _fit_all(samples, step):
    """Refit every entry's efficiencies; total squared log error."""
    total = 0.0
    fitted = {}
    for entry, smp in samples.items():
        if not smp:
            continue
        eff, eff1, rms = fit_entry(entry, smp, eff1_matters(entry), step)
        fitted[entry] = (eff, eff1, rms)
        total += rms * rms * len(smp)
    return total, fitted


def _objective(samples, n, report_path, step):
    """(mean squared log error of the model + mean log loss of the picks,
    rms log error, geometric-mean pick / fastest, worst pick / fastest,
    fitted efficiencies): the entries' efficiencies refitted first. The pick
    term is what the model is for: a lower error that makes the library pick
    slower entries is no better."""
    total, fitted = _fit_all(samples, step)
    rows, worst, geo = check_picks(report_path, write_md=False)
    return total / n - math.log(geo), math.sqrt(total / n), geo, worst, fitted


def _evaluate(samples, n, report_path):
    """_objective for the library as loaded (no refit): (objective, rms log
    error, geometric-mean pick / fastest, worst pick / fastest)."""
    total = 0.0
    for entry, smp in samples.items():
        for M, N, K, t in smp:
            total += math.log(fg.fg_estimate_seconds(M, N, K, entry) / t) ** 2
    rows, worst, geo = check_picks(report_path, write_md=False)
    return total / n - math.log(geo), math.sqrt(total / n), geo, worst


def fit_model(report_path, sweeps=2, write=True):
    """Host only: the cost model's shared constants (FIT_CONSTANTS) and the
    entries' efficiencies, fitted together to the search report's timings by
    coordinate descent on _objective (each constant tried at FIT_FACTORS of
    its current value with every entry's efficiencies refitted on a 0.02
    grid, two sweeps; then a final 0.01 fit). Writes csrc/fg_model.inc and
    csrc/fg_tuned.inc only if the fit beats the library as built (its
    compiled constants and efficiencies); records the comparison in the
    report either way and returns it."""
    fg.load_library()
    report = json.load(open(report_path))
    samples = model_samples(report)
    n = sum(len(v) for v in samples.values())
    j0, rms0, geo0, worst0 = _evaluate(samples, n, report_path)
    cur = {c: fg.fg_get_model_constant(c) for c in FIT_CONSTANTS}
    start = dict(cur)
    built_eff = {e: fg.fg_get_efficiency(e) for e in samples}
    best = _objective(samples, n, report_path, 0.02)[0]
    for sweep in range(sweeps):
        for c in FIT_CONSTANTS:
            base = cur[c]
            for f in FIT_FACTORS:
                v = base * f
                if fg.fg_set_model_constant(c, v) != fg.FG_OK:
                    continue
                j = _objective(samples, n, report_path, 0.02)[0]
                if j < best - 1e-12:
                    best, cur[c] = j, v
            fg.fg_set_model_constant(c, cur[c])
            print(f"[fit-model] sweep {sweep}: {c} = {cur[c]:.4g}, objective {best:.5f}",
                  flush=True)
    j1, rms1, geo1, worst1, fitted = _objective(samples, n, report_path, 0.01)
    result = {"constants": cur, "samples": n,
              "before": {"objective": j0, "rms_log_error": rms0, "geomean_pick": geo0,
                         "worst_pick": worst0, "constants": start},
              "after": {"objective": j1, "rms_log_error": rms1, "geomean_pick": geo1,
                        "worst_pick": worst1}}
    print(f"[fit-model] objective {j0:.5f} -> {j1:.5f}; rms log error {rms0:.4f} -> "
          f"{rms1:.4f}; picks (geo mean, worst) {geo0:.4f}, {worst0:.4f} -> {geo1:.4f}, "
          f"{worst1:.4f} over {n} timings", flush=True)
    if j1 >= j0:
        print("[fit-model] no improvement on the library as built; constants and "
              "efficiencies unchanged", flush=True)
        result["written"] = False
        # the loaded library's model back to what it was built with
        for c, v in start.items():
            fg.fg_set_model_constant(c, v)
        for e, (eff, eff1) in built_eff.items():
            fg.fg_set_efficiency(e, eff, eff1)
        if write:
            report["model_fit"] = result
            with open(report_path, "w") as f:
                json.dump(report, f)
        return result
    result["written"] = True
    rmsb, rmsa = rms0, rms1
    result["rms_log_error_before"], result["rms_log_error_after"] = rmsb, rmsa
    if write:
        lines = ["// Fitted constants of the cost model: FG_MODEL(fg_model_constant, value).",
                 "// Written by fp32_gemm_tile_amd/autotune.py --fit-model from the tile search's",
                 f"// timings ({n} timings of the table's entries, one MI355X, "
                 f"{report['date'][:10]}): rms log error",
                 f"// {rmsb:.4f} -> {rmsa:.4f}, the library's pick on the search shapes "
                 f"{geo0:.4f} -> {geo1:.4f} of the",
                 f"// fastest instance on geometric mean ({worst0:.4f} -> {worst1:.4f} at "
                 "worst). The split-K slice",
                 "// rate (FG_MODEL_SPLIT_BW) has no timing there and keeps its default."]
        for c in FIT_CONSTANTS:
            lines.append(f"FG_MODEL(FG_MODEL_{c.upper()}, {cur[c]:.6g})")
        with open(MODEL_INC, "w") as f:
            f.write("\n".join(lines) + "\n")
        old = open(INC_PATH).read().splitlines()
        new = []
        for l in old:
            m = re.match(r"\{(\w+), [0-9.]+, [0-9.]+\},(.*)", l)
            if m:
                key = m.group(1)
                eid = [c["id"] for c in fg.configs() if c["kind"] == fg.FG_KIND_SKINNY][0] \
                    if key == "FG_ID_SKINNY" else int(key)
                if eid in fitted:
                    eff, eff1, _ = fitted[eid]
                    l = f"{{{key}, {eff:.3f}, {eff1:.3f}}},{m.group(2)}"
            new.append(l)
        with open(INC_PATH, "w") as f:
            f.write("\n".join(new) + "\n")
        report["model_fit"] = result
        with open(report_path, "w") as f:
            json.dump(report, f)
    return result


REPORT_PATH = os.path.join(HERE, "tuning", "tile_search.json")
SEARCH_MD = os.path.join(ROOT, "profiles", "tile_search.md")
COVER_MARGIN = 0.01


def _report_times(report):
    """[(shape tuple, {instance id: seconds})] of a search report: the
    refined times where the refinement re-timed an instance, else the first
    pass."""
    out = []
    for r in report["shapes"]:
        t = {int(k): v for k, v in r["seconds"].items()}
        t.update({int(k): v for k, v in r.get("refined", {}).items()})
        out.append((tuple(r["shape"]), t))
    return out


def read_tuned_skinny(path=INC_PATH):
    """(eff, eff1) of the few-row row in a generated efficiency table, or None."""
    for line in open(path):
        line = line.split("//")[0].strip().rstrip(",")
        if line.startswith("{FG_ID_SKINNY,"):
            _, e, e1 = line.strip("{}").split(",")
            return float(e), float(e1)
    return None


def select_cover(report, margin=COVER_MARGIN):
    """Greedy cover: instances in the order they were kept, such that every
    search shape has a kept instance within `margin` of the fastest time
    measured on it by any instance (or the few-row entry is that fast).
    Each step keeps the instance that brings the most uncovered shapes within
    the margin, ties broken by the geometric-mean speed it adds."""
    inst = {r["id"]: r for r in report["instances"] if r["exact"]}
    times = _report_times(report)
    best = [min(t.values()) for _, t in times]
    sk = _skinny_id(report)
    covered = [sk in t and t[sk] <= (1 + margin) * b for (_, t), b in zip(times, best)]
    kept = []

    def cur_best(i, extra=None):
        ids = kept + ([extra] if extra is not None else [])
        vals = [times[i][1][k] for k in ids if k in times[i][1]]
        return min(vals) if vals else None

    while not all(covered):
        def score(c):
            gain = sum(1 for i, (_, t) in enumerate(times)
                       if not covered[i] and c in t and t[c] <= (1 + margin) * best[i])
            lg = 0.0
            for i in range(len(times)):
                b = cur_best(i, c)
                if b is not None:
                    lg += math.log(best[i] / b)
            return gain, lg
        c = max((c for c in inst if c not in kept), key=score)
        if score(c)[0] == 0:
            raise RuntimeError("no instance covers the remaining shapes")
        kept.append(c)
        covered = [cv or (c in t and t[c] <= (1 + margin) * best[i])
                   for i, (cv, (_, t)) in enumerate(zip(covered, times))]
    return kept


def select_from_report(report_path, write=True):
    """Keep a cover of the search shapes, assign table ids (the fixed rows
    stay at theirs), give each 16-byte-load entry a fallback for rows that
    are not 16-byte aligned, and write the instance list and efficiencies."""
    from fp32_gemm_tile_amd import build as fgbuild
    report = json.load(open(report_path))
    inst = {r["id"]: r for r in report["instances"]}
    kept = select_cover(report)
    anyalign = [k for k in kept if not needs_aligned_rows(inst[k])]
    if not anyalign:
        raise RuntimeError("the cover has no entry for rows that are not 16-byte aligned")
    ids = {k: n for n, k in enumerate(kept)}
    entries = []
    for k in kept:
        r = inst[k]
        e = {f: r[f] for f in fgbuild.ENTRY_FIELDS}
        e["id"] = ids[k]
        if needs_aligned_rows(r):
            # the any-alignment entry of the same tile if kept, else of the
            # nearest tile area
            same = [a for a in anyalign if (inst[a]["bm"], inst[a]["bn"]) == (r["bm"], r["bn"])]
            near = same or sorted(anyalign, key=lambda a: abs(math.log(
                inst[a]["bm"] * inst[a]["bn"] / (r["bm"] * r["bn"]))))
            e["fallback"] = ids[near[0]]
        else:
            e["fallback"] = -1
        entries.append(e)
    tuned = {ids[k]: (inst[k]["eff"], inst[k]["eff1"]) for k in kept}
    # the few-row entry keeps its fitted figures
    sk_old = read_tuned_skinny()
    if sk_old:
        tuned["FG_ID_SKINNY"] = sk_old
    if write:
        write_instance_list(
            INSTANCES_PATH, entries,
            "Matrix-core entries of the tile-configuration table, one kernel instance each\n"
            "(compiled from sgemm_mfma_inst.hip, one translation unit per line and layout).\n"
            "Written by fp32_gemm_tile_amd/autotune.py --select from the tile search's report\n"
            "(fp32_gemm_tile_amd/tuning/tile_search.json): the greedy cover of its shapes.")
        names = {ids[k]: inst[k]["name"] for k in kept}
        names["FG_ID_SKINNY"] = SKINNY
        lines = ["// Cost-model efficiencies of the modelled table entries: {id, eff, eff1}.",
                 "// eff: fraction of the fp32 matrix peak a wave reaches with its SIMD full;",
                 "// eff1: the same with one wave per SIMD (the few-row entry: eff divides",
                 "// its modelled step time, eff1 unused). Matrix-core rows: fitted by",
                 "// fp32_gemm_tile_amd/autotune.py --select from the tile search's timings",
                 f"// ({len(report['shapes'])} shapes, one MI355X, {report['date'][:10]})."]
        for i in sorted(tuned, key=lambda i: (isinstance(i, str), i if isinstance(i, int) else 0)):
            lines.append(f"{{{i}, {tuned[i][0]:.3f}, {tuned[i][1]:.3f}}},  // {names[i]}")
        with open(INC_PATH, "w") as f:
            f.write("\n".join(lines) + "\n")
    return entries, ids


def check_picks(report_path, write_md=True):
    """With the library built from the selected list: for every search shape,
    the speed of the entry the library picks (fg_select_config) relative to
    the fastest instance the search measured on it. Host only."""
    report = json.load(open(report_path))
    inst = {r["id"]: r for r in report["instances"]}
    by_key = {shape_key(r): r["id"] for r in report["instances"]}
    from fp32_gemm_tile_amd import build as fgbuild
    table = {e["id"]: e for e in fgbuild.read_instances(INSTANCES_PATH)}
    rows = []
    for sh, t in _report_times(report):
        M, N, K, ta, tb = sh[:5]
        lda, ldb, ldc = _lds(sh)
        pick = fg.fg_select_config(ta, tb, M, N, K, lda=lda, ldb=ldb, ldc=ldc)
        if pick["kind"] == fg.FG_KIND_SKINNY:
            rid = _skinny_id(report)
        else:
            e = table[pick["id"]]
            if needs_aligned_rows(e) and not _aligned(sh):
                e = table[e["fallback"]]
            rid = by_key[shape_key(e)]
        best = min(t, key=t.get)
        kept_ids = [by_key[shape_key(e)] for e in table.values()] + [_skinny_id(report)]
        kbest = min((k for k in kept_ids if k in t), key=t.get)
        rows.append({"shape": list(sh[:5]), "best": inst.get(best, {}).get("name", SKINNY),
                     "best_tflops": 2 * M * N * K / t[best] / 1e12,
                     "kept_best": inst.get(kbest, {}).get("name", SKINNY),
                     "pick": pick["name"], "pick_tflops": 2 * M * N * K / t[rid] / 1e12,
                     "pick_over_best": t[best] / t[rid], "kept_over_best": t[best] / t[kbest]})
    worst = min(r["pick_over_best"] for r in rows)
    geo = math.exp(sum(math.log(r["pick_over_best"]) for r in rows) / len(rows))
    if write_md:
        write_search_md(report, rows, worst, geo)
    return rows, worst, geo


def write_search_md(report, rows, worst, geo):
    from fp32_gemm_tile_amd import build as fgbuild
    inst = report["instances"]
    n_exact = sum(r["exact"] for r in inst)
    kept = fgbuild.read_instances(INSTANCES_PATH)
    L = ["# Tile search: instances, timings, kept set", "",
         f"One MI355X ({report['device']}), {report['date']}. Generated by "
         "`python -m fp32_gemm_tile_amd.autotune --select fp32_gemm_tile_amd/tuning/"
         "tile_search.json --check` from the report that", "",
         "    python -m fp32_gemm_tile_amd.autotune --build-search        # any host",
         "    python -m fp32_gemm_tile_amd.autotune --search <report>     # on the GPU", "",
         "wrote. Search space (`autotune.search_space`): workgroup tiles of "
         f"{len(TILES)} shapes from 64x64 to 256x256 with 4 or 8 waves, BK in {{8, 16, 32}}, "
         "32x32x2 or 16x16x4 MFMA blocks, 16- and 4-byte direct-to-LDS loads, the deepest "
         "ring (3 or 4) the LDS allows at the occupancy the registers allow, plus the "
         f"table's previous entries: {len(inst)} instances, {n_exact} bit-exact on the "
         "integer check (the rest: " + (", ".join(f"{r['name']} ({r['error']})"
                                                  for r in inst if not r["exact"]) or "none")
         + ").", "",
         f"Kept (greedy cover, every shape within {COVER_MARGIN:.0%} of the fastest instance): "
         f"{len(kept)} matrix-core entries. The library's pick runs at "
         f"{geo:.3f} of the fastest instance on geometric mean over {len(rows)} shapes, "
         f"{worst:.3f} at worst.", "",
         "| shape | fastest instance | TFLOP/s | library pick | TFLOP/s | pick / fastest |",
         "|---|---|---|---|---|---|"]
    for r in rows:
        M, N, K, ta, tb = r["shape"]
        L.append(f"| {M}x{N}x{K} {ta}{tb} | {r['best']} | {r['best_tflops']:.1f} | "
                 f"{r['pick']} | {r['pick_tflops']:.1f} | {r['pick_over_best']:.3f} |")
    L += ["", "Kept entries (table id, instance, waves per SIMD, fallback for unaligned rows):",
          ""]
    for e in kept:
        L.append(f"- {e['id']}: {instance_name(e)}, {e['wps']} waves/SIMD, "
                 f"fallback {e['fallback']}")
    L += ["", "Fastest time per instance relative to the fastest instance, geometric mean "
          "over the shapes each was timed on (all exact instances):", "",
          "| instance | shapes | speed vs fastest (geo mean) | eff | eff1 |", "|---|---|---|---|---|"]
    times = _report_times(report)
    for r in sorted(inst, key=lambda r: r["name"]):
        if not r["exact"]:
            continue
        ratios = [min(t.values()) / t[r["id"]] for _, t in times if r["id"] in t]
        if ratios:
            g = math.exp(sum(map(math.log, ratios)) / len(ratios))
            L.append(f"| {r['name']} | {len(ratios)} | {g:.3f} | {r.get('eff', '-')} | "
                     f"{r.get('eff1', '-')} |")
    with open(SEARCH_MD, "w") as f:
        f.write("\n".join(L) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--quick", action="store_true", help="a subset of the shapes")
    ap.add_argument("--write", action="store_true",
                    help="rewrite csrc/fg_tuned.inc with the fitted efficiencies")
    ap.add_argument("--report", default=None, help="JSON report path")
    ap.add_argument("--from-report", default=None,
                    help="no timing: take the fitted efficiencies from a saved report "
                         "(with --write, regenerate fg_tuned.inc from it)")
    ap.add_argument("--build-search", action="store_true",
                    help="write the search instance list and build the search library")
    ap.add_argument("--search", default=None, metavar="REPORT",
                    help="on the GPU: check and time every search instance, write REPORT")
    ap.add_argument("--refine", default=None, metavar="REPORT",
                    help="on the GPU: re-time the near-fastest instances of every shape of "
                         "REPORT (updates it)")
    ap.add_argument("--fit-model", default=None, metavar="REPORT",
                    help="host only: fit the cost model's shared constants and the entries' "
                         "efficiencies to REPORT's timings (rewrites csrc/fg_model.inc and "
                         "csrc/fg_tuned.inc)")
    ap.add_argument("--retime-few-rows", default=None, metavar="REPORT",
                    help="on the GPU: re-time the built library's few-row entry on the search "
                         "shapes of REPORT, refit its efficiency (updates REPORT and "
                         "csrc/fg_tuned.inc)")
    ap.add_argument("--select", default=None, metavar="REPORT",
                    help="keep a cover of the search shapes from REPORT; rewrite "
                         "csrc/fg_mfma_instances.inc and csrc/fg_tuned.inc")
    ap.add_argument("--check", default=None, metavar="REPORT",
                    help="with the library rebuilt from the selection: the pick on every "
                         "search shape against the fastest instance; writes "
                         "profiles/tile_search.md")
    args = ap.parse_args(argv)

    if args.build_search:
        build_search(verbose=False)
        return 0
    if args.search:
        run_search(args.search, QUICK if args.quick else None)
        return 0
    if args.refine:
        refine_search(args.refine)
        return 0
    if args.fit_model:
        fit_model(args.fit_model)
        return 0
    if args.retime_few_rows:
        retime_few_rows(args.retime_few_rows)
        return 0
    if args.select:
        entries, _ = select_from_report(args.select)
        print(f"[select] kept {len(entries)} entries; rebuild the library, then --check",
              flush=True)
        return 0
    if args.check:
        rows, worst, geo = check_picks(args.check)
        print(json.dumps({"shapes": len(rows), "geomean_pick_vs_fastest": geo,
                          "worst_pick_vs_fastest": worst}), flush=True)
        return 0

    if args.from_report:
        with open(args.from_report) as f:
            rep = json.load(f)
        fitted = {v["id"]: (v["eff"], v["eff1"], v["rms_log_error"])
                  for v in rep["fitted"].values()}
        if args.write:
            write_inc(fitted, rep["summary"]["shapes"])
            print(f"[autotune] wrote {INC_PATH} from {args.from_report}", flush=True)
        return 0

    import torch
    if not torch.cuda.is_available():
        print("autotune: no GPU visible", file=sys.stderr)
        return 1
    fg.load_library()
    shapes = QUICK if args.quick else SHAPES
    before = {e: fg.fg_get_efficiency(e) for e in range(fg.fg_num_configs())
              if fg.fg_get_config(e)["kind"] in (fg.FG_KIND_MFMA, fg.FG_KIND_SKINNY)}

    timings = []
    for sh in shapes:
        t = time_entries(sh, candidates(sh))
        timings.append((sh, t))
        best = min(t, key=t.get)
        print(f"[autotune] {sh[:5]} best {fg.fg_get_config(best)['name']} "
              f"{2 * sh[0] * sh[1] * sh[2] / t[best] / 1e12:.1f} TFLOP/s", flush=True)

    fitted = {}
    for e in before:
        few_rows = fg.fg_get_config(e)["kind"] == fg.FG_KIND_SKINNY
        samples = [(sh[0], sh[1], sh[2], t[e]) for sh, t in timings
                   if e in t and not (few_rows and sh[0] > 256)]
        if samples:
            fitted[e] = fit_entry(e, samples, eff1_matters(e))
        else:
            fitted[e] = (*before[e], float("nan"))

    picks = []
    for sh, t in timings:
        M, N, K, ta, tb = sh[:5]
        lda, ldb, ldc = _lds(sh)
        pick = fg.fg_select_config(ta, tb, M, N, K, lda=lda, ldb=ldb, ldc=ldc)["id"]
        best = min(t, key=t.get)
        ratio = t[best] / t[pick] if pick in t else None
        picks.append({"shape": list(sh[:5]), "best": fg.fg_get_config(best)["name"],
                      "pick": fg.fg_get_config(pick)["name"],
                      "pick_over_best_speed": ratio,
                      "seconds": {fg.fg_get_config(e)["name"]: v for e, v in t.items()}})
    ratios = [p["pick_over_best_speed"] for p in picks if p["pick_over_best_speed"]]
    summary = {"shapes": len(timings),
               "geomean_pick_speed_vs_best": math.exp(sum(map(math.log, ratios)) / len(ratios)),
               "worst_pick_speed_vs_best": min(ratios)}
    report = {"date": datetime.datetime.now().isoformat(timespec="seconds"),
              "fitted": {fg.fg_get_config(e)["name"]: {"id": e, "eff": v[0], "eff1": v[1],
                                                       "rms_log_error": v[2]}
                         for e, v in fitted.items()},
              "before": {fg.fg_get_config(e)["name"]: list(v) for e, v in before.items()},
              "summary": summary, "picks": picks}
    print(json.dumps(summary), flush=True)
    if args.report:
        with open(args.report, "w") as f:
            json.dump(report, f, indent=1)
    if args.write:
        write_inc(fitted, len(timings))
        print(f"[autotune] wrote {INC_PATH}; rebuild the library to use it", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
