"""Offline tuner for the tile-configuration table.

The library picks a table entry per call with a cost model (fg_api.cpp) that
holds, for every matrix-core entry, two efficiencies: ``eff`` (fraction of
the fp32 matrix peak a wave reaches with its SIMD full) and ``eff1`` (the same
with one wave per SIMD); the few-row entry has one, dividing its modelled
time per step of K. This module measures every entry on a grid of shapes
on the GPU it runs on, fits the two efficiencies of each entry to those
timings, checks that the refitted model's picks agree with the measured
best, and with ``--write`` regenerates ``csrc/fg_tuned.inc`` (rebuild the
library afterwards) and a JSON report.

This is the empirical configuration search of "How to get a matmul kernel
into the top percentile (worklog)", section "Extra" (the configuration found
for one GPU is retuned for another) and of "Matmul II: register blocking,
warp tiling, tensor cores", section 8 (many kernel variants and a heuristic
that picks one per call), done per shape class on an MI355X.

Usage (on the GPU):
    python -m fp32_gemm_tile_amd.autotune [--quick] [--write] [--report PATH]
and, on any host, from a saved report:
    python -m fp32_gemm_tile_amd.autotune --from-report PATH --write
"""
from __future__ import annotations

import argparse
import datetime
import json
import math
import os
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
            if not _aligned(shape) and c["name"].endswith(("_s4", "_s3")):
                continue
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


def fit_entry(entry, samples, wps_gt_1):
    """Efficiencies of one modelled entry that minimise the squared log
    error of the model against `samples` = [(M, N, K, seconds), ...]: a grid
    search over eff in [0.30, 1.00] and, when several waves can share a SIMD,
    eff1 in [0.20, eff] (steps of 0.01). Leaves the library holding the
    best pair; returns (eff, eff1, rms log error)."""
    best = None
    effs = [round(0.30 + 0.01 * i, 2) for i in range(71)]
    for eff in effs:
        ones = [round(0.20 + 0.01 * i, 2) for i in range(int(round((eff - 0.20) / 0.01)) + 1)] \
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
        lines.append(f"{{{e}, {eff:.3f}, {eff1:.3f}}},  // {fg.fg_get_config(e)['name']}")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--quick", action="store_true", help="a subset of the shapes")
    ap.add_argument("--write", action="store_true",
                    help="rewrite csrc/fg_tuned.inc with the fitted efficiencies")
    ap.add_argument("--report", default=None, help="JSON report path")
    ap.add_argument("--from-report", default=None,
                    help="no timing: take the fitted efficiencies from a saved report "
                         "(with --write, regenerate fg_tuned.inc from it)")
    args = ap.parse_args(argv)

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
