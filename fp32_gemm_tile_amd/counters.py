"""Hardware-counter evidence for one workload of the bench: a kernel trace and
separate rocprofv3 counter passes, summarised per GEMM kernel.

Each pass is its own run of ``bench.py`` under ``rocprofv3`` (the bench is the
program after ``--``; counter passes never combine with tracing), bounded by
``timeout -s KILL``:

  trace   --kernel-trace --stats             average kernel duration
  fetch   --pmc FETCH_SIZE                   HBM bytes read (KiB per dispatch)
  write   --pmc WRITE_SIZE                   HBM bytes written
  mfma    --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
                SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_BUSY_CYCLES
  lds     --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS
                SQ_WAIT_INST_LDS
  wait    --pmc SQ_WAIT_ANY SQ_WAVE_CYCLES SQ_WAVES SQ_INSTS_VALU

The fetch and write passes end with three plain device copies of 1 GiB
(``bench.py --copy-probe``), whose counter values give the scale from
FETCH_SIZE / WRITE_SIZE to bytes. Derived figures:

  MfmaUtil   = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs)
  MFMA FLOP  = SQ_INSTS_VALU_MFMA_MOPS_F32 x 512
  conflicts  = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles per active cycle)
  wait share = SQ_WAIT_ANY / SQ_WAVE_CYCLES

Usage (on the GPU machine, from the repository root):
    python -m fp32_gemm_tile_amd.counters --workload C3 --out gpurun_out/counters_C3 \
        [--config ID] [--group-m G] [--xcd-remap 0|1] [--ops NN|NT|TN|TT]
        [--passes trace fetch ...]
    python -m fp32_gemm_tile_amd.counters --summarize gpurun_out/counters_C3
    python -m fp32_gemm_tile_amd.counters --out gpurun_out/bench_trace --bench-trace [ARGS]
(the last: bench.py with ARGS -- none for its default run -- under the
kernel trace, summarised per kernel and launch size). The summary (Markdown, with the commands) is printed and written to
``<out>/summary.md`` and ``<out>/summary.json``.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shlex
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PASSES = {
    "trace": ["--kernel-trace", "--stats"],
    "fetch": ["--pmc", "FETCH_SIZE"],
    "write": ["--pmc", "WRITE_SIZE"],
    "mfma": ["--pmc", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE",
             "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_BUSY_CYCLES"],
    "lds": ["--pmc", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS",
            "SQ_WAIT_INST_LDS"],
    "wait": ["--pmc", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES", "SQ_WAVES", "SQ_INSTS_VALU"],
}
COPY_KERNEL = "copyBuffer"
SIMDS = 1024
XCDS = 8


def bench_args(a):
    out = ["--workload", a.workload, "--steps", str(a.steps), "--warmup", str(a.warmup),
           "--no-cpu", "--no-probes", "--no-extras"]
    if a.config >= 0:
        out += ["--config", str(a.config)]
    if a.group_m:
        out += ["--group-m", str(a.group_m)]
    if a.xcd_remap != 1:
        out += ["--xcd-remap", str(a.xcd_remap)]
    for flag in ("splitk", "streamk"):
        if getattr(a, flag):
            out.append(f"--{flag}")
    if a.ops:
        out += ["--ops", a.ops]
    return out


def run_pass(name, a, out_dir):
    """One rocprofv3 run of the bench; returns the command (as a string)."""
    d = os.path.join(out_dir, name)
    cmd = ["timeout", "-s", "KILL", str(a.timeout), "rocprofv3", *PASSES[name],
           "--output-format", "csv", "-d", d, "-o", "run", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *bench_args(a)]
    if name in ("fetch", "write"):
        cmd.append("--copy-probe")
    print(f"[counters] {a.workload} pass {name}", flush=True)
    env = dict(os.environ, TMPDIR="/tmp")
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True)
    with open(os.path.join(out_dir, f"{name}.log"), "w") as f:
        f.write(r.stdout + "\n---- stderr ----\n" + r.stderr)
    bench_line = [l for l in r.stdout.splitlines() if l.startswith("{")]
    # rocprofv3 may end with a signal after the program has finished and its
    # files are complete; the program's own last line says whether it ran.
    if not bench_line:
        raise RuntimeError(f"pass {name} failed (rc {r.returncode}); see {name}.log")
    with open(os.path.join(out_dir, f"{name}.bench.json"), "w") as f:
        f.write(bench_line[-1] + "\n")
    return " ".join(shlex.quote(c) for c in cmd).replace(ROOT, "$REPO")


def _rows(pattern):
    rows = []
    for path in glob.glob(pattern, recursive=True):
        with open(path, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def counters(out_dir, name):
    """{kernel name: {counter: mean value per dispatch}} of one pass, plus the
    number of dispatches and grid size per kernel."""
    per = {}
    for r in _rows(os.path.join(out_dir, name, "**", "*counter_collection.csv")):
        k = r.get("Kernel_Name", "")
        d = per.setdefault(k, {"dispatches": set(), "values": {}})
        d["dispatches"].add(r.get("Dispatch_Id"))
        d["grid"] = int(float(r.get("Grid_Size", 0) or 0))
        d["values"].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = {}
    for k, d in per.items():
        n = max(1, len(d["dispatches"]))
        out[k] = {c: sum(v) / n for c, v in d["values"].items()}
        out[k]["_dispatches"] = n
        out[k]["_grid"] = d.get("grid", 0)
    return out


def kernel_stats(out_dir):
    out = {}
    for r in _rows(os.path.join(out_dir, "trace", "**", "*kernel_stats.csv")):
        out[r["Name"]] = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                          "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3}
    return out


def dispatches(out_dir, pass_name="trace"):
    """Per (kernel, launch size in work-items) of a kernel-trace pass: calls
    and mean / median / min / max duration (us)."""
    import statistics
    groups = {}
    for r in _rows(os.path.join(out_dir, pass_name, "**", "*kernel_trace.csv")):
        n = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((r["Kernel_Name"], n), []).append(d)
    return {k: {"calls": len(v), "avg_us": sum(v) / len(v), "median_us": statistics.median(v),
                "min_us": min(v), "max_us": max(v)} for k, v in groups.items()}


def bench_trace(out_dir, bench_argv, timeout):
    """The bench as given (default: its default run) under rocprofv3's kernel
    trace; a summary of every GEMM kernel per launch size beside the bench's
    own line, whose mean time per call must agree with the trace's average
    for the kernel and size it reports."""
    os.makedirs(out_dir, exist_ok=True)
    d = os.path.join(out_dir, "trace")
    cmd = ["timeout", "-s", "KILL", str(timeout), "rocprofv3", "--kernel-trace", "--stats",
           "--output-format", "csv", "-d", d, "-o", "run", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *bench_argv]
    print("[counters] bench under the kernel trace", flush=True)
    r = subprocess.run(cmd, cwd="/tmp", env=dict(os.environ, TMPDIR="/tmp"), capture_output=True,
                       text=True)
    with open(os.path.join(out_dir, "trace.log"), "w") as f:
        f.write(r.stdout + "\n---- stderr ----\n" + r.stderr)
    line = [l for l in r.stdout.splitlines() if l.startswith("{")]
    if not line:
        raise RuntimeError(f"bench under the trace failed (rc {r.returncode}); see trace.log")
    b = json.loads(line[-1])
    disp = dispatches(out_dir)
    cmdline = " ".join(shlex.quote(c) for c in cmd).replace(ROOT, "$REPO")
    L = ["Command (from the repository root `$REPO`, run from /tmp):", "", f"    {cmdline}", "",
         f"Bench line: value {b['value']} {b['unit']}, ms_per_step {b['ms_per_step']} "
         f"(workload {b['config']['workload']}, entry {b['config']['kernel_config']}).", "",
         "| kernel | work-items per launch | calls | avg (us) | median (us) | min (us) | max (us) |",
         "|---|---|---|---|---|---|---|"]
    for (k, n), v in sorted(disp.items(), key=lambda kv: -kv[1]["calls"] * kv[1]["avg_us"]):
        if COPY_KERNEL in k or not ("fg::" in k or "gemm" in k.lower()):
            continue
        L.append(f"| `{k}` | {n} | {v['calls']} | {v['avg_us']:.1f} | {v['median_us']:.1f} | "
                 f"{v['min_us']:.1f} | {v['max_us']:.1f} |")
    cfg = b["config"]
    flops = 2.0 * cfg["M"] * cfg["N"] * cfg["K"]
    head = max((kv for kv in disp.items() if "fg::" in kv[0][0]),
               key=lambda kv: kv[1]["calls"] * kv[1]["avg_us"], default=None)
    if head:
        (k, n), v = head
        L += ["", f"Dominant kernel `{k}` ({n} work-items): trace average {v['avg_us']:.1f} us "
              f"= {flops / (v['avg_us'] * 1e-6) / 1e12:.2f} TFLOP/s; the bench's "
              f"ms_per_step {b['ms_per_step'] * 1e3:.1f} us "
              f"(ratio {b['ms_per_step'] * 1e3 / v['avg_us']:.4f}).", ""]
    md = "\n".join(L) + "\n"
    with open(os.path.join(out_dir, "trace_summary.md"), "w") as f:
        f.write(md)
    return md


def _gemm_kernel(table):
    """The GEMM kernel of a pass: the one with the most dispatches among
    those that are not the copy probe, nor torch's own fill/rand kernels."""
    cands = {k: v for k, v in table.items()
             if COPY_KERNEL not in k and ("fg::" in k or "sgemm" in k or "gemm" in k.lower())}
    if not cands:
        return None
    return max(cands, key=lambda k: (cands[k].get("_dispatches", cands[k].get("calls", 0)),
                                     cands[k].get("_grid", 0)))


def summarize(out_dir):
    meta = json.load(open(os.path.join(out_dir, "meta.json")))
    bench = {}
    for p in PASSES:
        path = os.path.join(out_dir, f"{p}.bench.json")
        if os.path.exists(path):
            bench[p] = json.load(open(path))
    res = {"workload": meta["workload"], "commands": meta["commands"]}
    stats = kernel_stats(out_dir) if "trace" in meta["commands"] else {}
    k = _gemm_kernel(stats) if stats else None
    any_bench = next(iter(bench.values()), {})
    cfg = any_bench.get("config", {})
    flops = 2.0 * cfg.get("M", 0) * cfg.get("N", 0) * cfg.get("K", 0)
    res["kernel_config"] = cfg.get("kernel_config")
    res["shape"] = {x: cfg.get(x) for x in ("M", "N", "K", "transA", "transB", "alpha", "beta")}
    if k:
        s = stats[k]
        res["kernel"] = k
        res["trace"] = dict(s, tflops=flops / (s["avg_us"] * 1e-6) / 1e12 if flops else None)
        res["bench_ms_per_step"] = bench.get("trace", {}).get("ms_per_step")
    copy_scale = {}
    for p, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        if p not in meta["commands"]:
            continue
        t = counters(out_dir, p)
        copy = next((v for kk, v in t.items() if COPY_KERNEL in kk), None)
        g = _gemm_kernel(t)
        if copy and ctr in copy:
            copy_scale[ctr] = (1 << 30) / (copy[ctr] * 1024.0)
        if g:
            res.setdefault("counters", {})[ctr + "_KiB"] = t[g][ctr]
            res.setdefault("kernel", g)
    if copy_scale:
        res["copy_scale"] = copy_scale
        c = res.get("counters", {})
        if "FETCH_SIZE_KiB" in c and "FETCH_SIZE" in copy_scale:
            res["hbm_read_bytes"] = c["FETCH_SIZE_KiB"] * 1024 * copy_scale["FETCH_SIZE"]
        if "WRITE_SIZE_KiB" in c and "WRITE_SIZE" in copy_scale:
            res["hbm_write_bytes"] = c["WRITE_SIZE_KiB"] * 1024 * copy_scale["WRITE_SIZE"]
    for p in ("mfma", "lds", "wait"):
        if p not in meta["commands"]:
            continue
        t = counters(out_dir, p)
        g = _gemm_kernel(t)
        if g:
            res.setdefault("counters", {}).update(
                {kk: v for kk, v in t[g].items() if not kk.startswith("_")})
    c = res.get("counters", {})
    if c.get("GRBM_GUI_ACTIVE"):
        res["mfma_util"] = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (
            c["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
    if "SQ_INSTS_VALU_MFMA_MOPS_F32" in c:
        res["mfma_flop"] = c["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512
        res["mfma_flop_over_2mnk"] = res["mfma_flop"] / flops if flops else None
    if c.get("SQ_LDS_IDX_ACTIVE"):
        res["lds_conflicts_per_active_cycle"] = c.get("SQ_LDS_BANK_CONFLICT", 0) / \
            c["SQ_LDS_IDX_ACTIVE"]
    if c.get("SQ_WAVE_CYCLES"):
        res["wait_share"] = c.get("SQ_WAIT_ANY", 0) / c["SQ_WAVE_CYCLES"]
    comp = 4.0 * (cfg.get("M", 0) * cfg.get("K", 0) + cfg.get("K", 0) * cfg.get("N", 0) +
                  cfg.get("M", 0) * cfg.get("N", 0) * (1 + (cfg.get("beta", 0) != 0)))
    res["compulsory_bytes"] = comp
    if "hbm_read_bytes" in res and "trace" in res:
        tot = res["hbm_read_bytes"] + res.get("hbm_write_bytes", 0)
        res["hbm_bytes"] = tot
        res["hbm_gbs"] = tot / (res["trace"]["avg_us"] * 1e-6) / 1e9
        res["hbm_over_compulsory"] = tot / comp if comp else None
    with open(os.path.join(out_dir, "summary.json"), "w") as f:
        json.dump(res, f, indent=1)
    if "hbm_read_bytes" in res and "hbm_write_bytes" in res:
        # the record bench.py reads for roofline.traffic (valid while the
        # kernel sources hash to the same value)
        sys.path.insert(0, ROOT)
        import bench
        rec = {"workload": meta["workload"], "kernel": res.get("kernel"),
               "kernel_config": res.get("kernel_config"),
               "kernel_source_sha": bench.kernel_source_sha(res.get("kernel_config") or "mfma_"),
               "fetch_kib_per_dispatch": res["counters"]["FETCH_SIZE_KiB"],
               "write_kib_per_dispatch": res["counters"]["WRITE_SIZE_KiB"],
               "fetch_scale": res["copy_scale"]["FETCH_SIZE"],
               "write_scale": res["copy_scale"]["WRITE_SIZE"],
               "bytes_per_launch": int(round(res["hbm_read_bytes"] + res["hbm_write_bytes"])),
               "source": f"profiles/counters_{meta['workload']}.md"}
        with open(os.path.join(out_dir, f"traffic_{meta['workload']}.json"), "w") as f:
            json.dump(rec, f, indent=1)
    md = render(res)
    with open(os.path.join(out_dir, "summary.md"), "w") as f:
        f.write(md)
    return res, md


def _f(v, fmt):
    return "-" if v is None else format(v, fmt)


def render(res):
    sh = res["shape"]
    lines = [f"### {res['workload']}: {sh['M']}x{sh['N']}x{sh['K']} "
             f"{sh['transA']}{sh['transB']}, entry {res.get('kernel_config')}", ""]
    t = res.get("trace", {})
    lines.append("| kernel avg (us) | TFLOP/s (trace) | MfmaUtil | MFMA FLOP / 2MNK | "
                 "LDS conflict cycles / active | wait share | HBM bytes / launch | "
                 "x compulsory | HBM GB/s |")
    lines.append("|---|---|---|---|---|---|---|---|---|")
    lines.append("| " + " | ".join([
        _f(t.get("avg_us"), ".1f"), _f(t.get("tflops"), ".1f"),
        _f(res.get("mfma_util"), ".1%"), _f(res.get("mfma_flop_over_2mnk"), ".4f"),
        _f(res.get("lds_conflicts_per_active_cycle"), ".3f"), _f(res.get("wait_share"), ".1%"),
        _f(res.get("hbm_bytes"), ".4g"), _f(res.get("hbm_over_compulsory"), ".2f"),
        _f(res.get("hbm_gbs"), ".0f")]) + " |")
    lines.append("")
    c = res.get("counters", {})
    if c:
        lines.append("Raw counters per dispatch: " + ", ".join(
            f"{k} {v:.4g}" for k, v in sorted(c.items())) + ".")
        lines.append("")
    if res.get("copy_scale"):
        lines.append("Copy-probe scale (bytes per counted byte): " + ", ".join(
            f"{k} x{v:.3f}" for k, v in res["copy_scale"].items()) + ".")
        lines.append("")
    lines.append(f"Kernel: `{res.get('kernel')}`.")
    lines.append("")
    lines.append("Commands (from the repository root `$REPO`, run from /tmp):")
    lines.append("")
    for p, cmd in res["commands"].items():
        lines.append(f"    {cmd}")
    lines.append("")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="C5a")
    ap.add_argument("--out", default=None)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=-1)
    ap.add_argument("--group-m", type=int, default=0)
    ap.add_argument("--xcd-remap", type=int, choices=(0, 1), default=1)
    ap.add_argument("--splitk", action="store_true")
    ap.add_argument("--streamk", action="store_true")
    ap.add_argument("--ops", choices=("NN", "NT", "TN", "TT"), default=None,
                    help="operand layouts instead of the workload's (bench.py --ops)")
    ap.add_argument("--passes", nargs="+", default=list(PASSES), choices=list(PASSES))
    ap.add_argument("--timeout", type=int, default=150, help="seconds per pass (SIGKILL)")
    ap.add_argument("--summarize", default=None, help="only summarise an existing directory")
    ap.add_argument("--bench-trace", nargs=argparse.REMAINDER, default=None, metavar="BENCH_ARG",
                    help="run bench.py with these arguments (none: its default run) under "
                         "the kernel trace and summarise per kernel and launch size into --out")
    a = ap.parse_args(argv)
    if a.bench_trace is not None:
        out = os.path.abspath(a.out or os.path.join(ROOT, "gpurun_out", "bench_trace"))
        print(bench_trace(out, a.bench_trace, max(a.timeout, 600)), flush=True)
        return 0
    if a.summarize:
        res, md = summarize(a.summarize)
        print(md)
        return 0
    # with --ops the records are named for the workload and the layouts
    # (bench.py reads traffic records of the workloads as defined only)
    name = a.workload + (f"_{a.ops}" if a.ops else "")
    out = os.path.abspath(a.out or os.path.join(ROOT, "gpurun_out", f"counters_{name}"))
    os.makedirs(out, exist_ok=True)
    meta = {"workload": name, "commands": {}}
    for p in a.passes:
        meta["commands"][p] = run_pass(p, a, out)
        with open(os.path.join(out, "meta.json"), "w") as f:
            json.dump(meta, f, indent=1)
    res, md = summarize(out)
    print(md, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
