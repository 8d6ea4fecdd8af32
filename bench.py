#!/usr/bin/env python3
"""SGEMM throughput on one MI355X: TFLOP/s and fraction of the fp32 peak.

Default workload: 8192 x 8192 x 8192 row-major NN, A and B uniform[-1,1)
from seed 4, alpha = 1, beta = 0 (the headline compute-bound shape). One
"step" is one full SGEMM call through the C ABI (fg_sgemm). Inputs are
resident in device memory before timing starts.

Prints ONE JSON line (rank 0) with the metric, the roofline of the dominant
kernel (timed with HIP events on the stream the kernel is launched on) and
the CPU oracle timed on the whole workload, with every element of the timed
result checked against it.

With the default workload it also times 4096^3 NN and the 1024 x 8192 x 8192
row block one of eight GPUs would own, and measures the device's attainable
MFMA and HBM-read rates with the library's probe kernels.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C5a]
                       [--suite] [--calibrate] [--splitk [S]] [--streamk] [--cold]
                       [--no-cpu] [--no-probes] [--no-extras] [--copy-probe]
                       [--config ID] [--group-m G] [--xcd-remap 0|1]
                       [--epilogue ACT] [--quant bf16|int8_row] [--launch-floor]
                       [--ops NN|NT|TN|TT]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3  # MI355X dense fp32 matrix peak (256 CU x 2.4 GHz x 256 FLOP/clk)
HBM_PEAK_GBS = 8000.0
METRIC = "fp32 SGEMM TFLOP/s and % of MI355X fp32 peak at 4096^3 and 8192^3"


def kernel_source_sha(kernel_config="mfma_"):
    """Hash of the sources that define the kernel family of a table entry
    (matrix-core, few-row or vector-ALU kernel) and its launch."""
    if kernel_config == "few_rows":
        family = "sgemm_skinny.hip"
    elif kernel_config.startswith("valu_"):
        family = "sgemm_valu.hip"
    else:
        family = "sgemm_mfma.h"
    h = hashlib.sha256()
    for f in (family, "fg_device.h", "fg_kernels.h"):
        with open(os.path.join(ROOT, "fp32_gemm_tile_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel_config):
    """Measured HBM traffic per launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel sources with the same table
    entry; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha(kernel_config):
        return None
    if t.get("kernel_config") not in (None, kernel_config):
        return None
    return t.get("bytes_per_launch")


def time_gpu(w, steps, warmup, config=-1, splitk=False, cold=False, sample_clock=False,
             epilogue=None, streamk=False, min_warm_s=0.0, keep_output=False, quant=None):
    """Time `steps` calls on the current stream with a HIP event pair around
    each call. Warm (default): the calls run back to back and the mean is the
    whole range over `steps`. Cold: a 512 MiB device write runs before each
    call (outside its event pair) so the operands start outside the caches."""
    import statistics

    import torch
    import fp32_gemm_tile_amd as fg
    from fp32_gemm_tile_amd import workloads as wl

    A, B, C = wl.make_inputs(w)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    dC = torch.from_numpy(C).cuda() if C is not None else torch.empty(
        (w.M, w.LDC), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    ws = torch.empty(64 << 20, dtype=torch.float32, device="cuda") if splitk else None
    nsplit = int(splitk) if splitk and not isinstance(splitk, bool) else 0
    flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda") if cold else None
    sk_ws, sk_bytes = None, 0
    if streamk:
        sk_bytes = fg.fg_sgemm_streamk_workspace_size(w.transA, w.transB, w.M, w.N, w.K,
                                                      dA.data_ptr(), w.LDA, dB.data_ptr(), w.LDB)
        sk_ws = torch.empty(max(sk_bytes, 16) // 4, dtype=torch.float32, device="cuda")
    qdesc, qbuf = None, None
    if quant is not None:
        # Q in its own buffer, rows aligned to 4 elements; int8 factors of
        # order 127 / max |C| for these inputs (the codes' values do not
        # change the work)
        esize = 2 if quant == "bf16" else 1
        qbuf = torch.empty(w.M * w.N * esize + 16, dtype=torch.uint8, device="cuda")
        qs = torch.full((w.M,), 127.0 / max(1.0, 0.6 * w.K ** 0.5), device="cuda")
        qdesc = fg.make_quant(quant, qbuf.data_ptr(), w.N, qs.data_ptr())
    epi = None
    if epilogue is not None:
        # every vector present: the most work the fused epilogue can do
        g = torch.Generator().manual_seed(w.seed)
        vecs = [torch.rand(n, generator=g).cuda() + 0.5 for n in (w.M, w.N)] + \
               [torch.randn(n, generator=g).cuda() for n in (w.M, w.N)]
        epi = fg.make_epilogue(*[v.data_ptr() for v in vecs], epilogue)

    def step():
        if splitk:
            st = fg.fg_sgemm_splitk(w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(),
                                    w.LDA, dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC,
                                    nsplit, ws.data_ptr(), ws.numel() * 4, sp)
        elif streamk:
            st = fg.fg_sgemm_streamk(w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(),
                                     w.LDA, dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC,
                                     sk_ws.data_ptr(), sk_bytes, sp)
        elif qdesc is not None:
            st = fg.fg_sgemm_quant(w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(),
                                   w.LDA, dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC,
                                   epi, qdesc, sp, config)
        elif epi is not None:
            st = fg.fg_sgemm_fused(w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(),
                                   w.LDA, dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC,
                                   epi, sp, config)
        else:
            st = fg.fg_sgemm_ex(w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(),
                                w.LDA, dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC,
                                sp, config)
        if st != 0:
            raise fg.FgError(st, fg.fg_last_bad_arg(), fg.fg_last_error())

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Tables of many short runs (--suite, --calibrate) keep calling until
    # min_warm_s has passed: after the host-side set-up between runs the GPU
    # idles, and a few short calls do not bring its clock back up.
    t_warm = time.perf_counter()
    while min_warm_s > 0 and time.perf_counter() - t_warm < min_warm_s:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    # Per-call event pairs (for the median and the minimum). Their records sit
    # between the calls, so the warm mean comes from a second pass with one
    # event pair around all `steps` calls.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        if cold:
            flush.fill_(float(i))
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    if cold:
        mean, wall = sum(per) / steps, None
    else:
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        mean = ev0.elapsed_time(ev1) / steps
    clock = None
    if sample_clock:
        # Outside the timed ranges: amd-smi samples the shader clock once a
        # second while about five seconds of the same calls run.
        watcher = start_clock_watch(seconds=4)
        if watcher is not None:
            time.sleep(1.0)
            for _ in range(int(min(4000, max(10, 5000.0 / max(mean, 1e-3))))):
                step()
            torch.cuda.synchronize()
            clock = finish_clock_watch(watcher)
    # The entry (and split-K slices) the timed call ran: fg_sgemm_splitk
    # takes no entry id and chooses with the split allowed; the stream-K line
    # names the entry of its data-parallel rounds.
    nsl = 1
    if splitk:
        cfg, nsl = fg.fg_select_config_ex(w.transA, w.transB, w.M, w.N, w.K, dA.data_ptr(),
                                          w.LDA, dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(),
                                          w.LDC, splits=nsplit, workspace_bytes=ws.numel() * 4)
    elif config >= 0:
        cfg = fg.fg_get_config(config)
    else:
        cfg = fg.fg_select_config_ex(w.transA, w.transB, w.M, w.N, w.K, dA.data_ptr(), w.LDA,
                                     dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC,
                                     quant=quant)[0]
    output = None
    if keep_output and epilogue is None:
        # Outside every timed range: one more call on the original C (with
        # beta != 0 the timed calls kept updating C), read back for the
        # element-wise check against the oracle.
        if C is not None:
            dC.copy_(torch.from_numpy(C))
        step()
        torch.cuda.synchronize()
        output = dC.cpu().numpy()[:, :w.N]
    return {"ms_per_launch": mean, "ms_median": statistics.median(per), "ms_min": min(per),
            "wall_s": wall, "config": cfg["name"], "splits": nsl, "clock_mhz": clock,
            "output": output}


def launch_floor(name, steps):
    """Per-call time of the smallest kernel the library launches: fg_sgemm
    with alpha = beta = 0 on the workload's C (C = 0, A and B unread), back to
    back after a 0.2 s warm-up; the same event pair as time_gpu."""
    import torch
    import fp32_gemm_tile_amd as fg
    from fp32_gemm_tile_amd import workloads as wl
    w = wl.WORKLOADS[name]
    dC = torch.empty((w.M, w.LDC), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        st = fg.fg_sgemm(w.transA, w.transB, w.M, w.N, w.K, 0.0, 0, w.LDA, 0, w.LDB, 0.0,
                         dC.data_ptr(), w.LDC, stream.cuda_stream)
        if st != 0:
            raise fg.FgError(st, fg.fg_last_bad_arg(), fg.fg_last_error())
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        for _ in range(16):
            step()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    return {"workload": name, "launch_floor_us": round(us, 3), "steps": steps,
            "call": "fg_sgemm, alpha = beta = 0 (C = 0: one fill kernel)"}


def measured_peaks():
    """The device's attainable fp32 MFMA rate and HBM read rate, from the
    library's probe kernels (an MFMA-only loop; a 2 GiB streaming read, far
    larger than the caches), best of five launches each."""
    import torch
    import fp32_gemm_tile_amd as fg

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    wgs, iters = 2048, 20000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    n = 1 << 29
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    rwgs = 512  # the best of 512 .. 16384 workgroups in a sweep on one MI355X
    rout = torch.empty(rwgs * 4, dtype=torch.float32, device="cuda")

    def best(launch):
        launch()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        return min(times)

    def mfma():
        if fg.fg_probe_mfma(wgs, iters, out.data_ptr(), sp) != 0:
            raise fg.FgError(fg.FG_ERR_HIP, 0, fg.fg_last_error())

    def read():
        if fg.fg_probe_read(x.data_ptr(), n, rwgs, rout.data_ptr(), sp) != 0:
            raise fg.FgError(fg.FG_ERR_HIP, 0, fg.fg_last_error())

    t_mfma = best(mfma)
    t_read = best(read)
    return {"mfma_tflops": round(fg.fg_probe_mfma_flops(wgs, iters) / t_mfma / 1e12, 2),
            "hbm_read_gbs": round(4.0 * n / t_read / 1e9, 1),
            "probes": "fg_probe_mfma 2048 WG x 20000 iterations; fg_probe_read of 2 GiB; "
                      "best of 5"}


def start_clock_watch(seconds):
    """Start amd-smi sampling the clocks once a second for `seconds` seconds
    (None if amd-smi cannot be started)."""
    import subprocess
    try:
        return subprocess.Popen(["amd-smi", "metric", "--clock", "--json", "-w", "1",
                                 "-W", str(seconds)], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None


def finish_clock_watch(proc):
    """Shader clock samples (MHz, mean over the XCDs of each sample) that
    amd-smi printed: the median and the maximum, or None."""
    import re
    import statistics
    import subprocess
    try:
        out, _ = proc.communicate(timeout=60)
    except subprocess.TimeoutExpired:
        proc.kill()
        return None
    vals = [float(v) for v in
            re.findall(r'"gfx_\d+":\s*\{\s*"clk":\s*\{\s*"value":\s*(\d+(?:\.\d+)?)', out)]
    if not vals:
        return None
    # eight XCDs per sample
    per_sample = [sum(vals[i:i + 8]) / len(vals[i:i + 8]) for i in range(0, len(vals), 8)]
    return {"median": round(statistics.median(per_sample), 1), "max": round(max(per_sample), 1),
            "samples": len(per_sample), "source": "amd-smi metric --clock, 1 s interval"}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, gpu_out=None, block=1024):
    """The oracle as it is, on the whole workload (every row of C), timed on
    the host's cores; with `gpu_out` (the timed calls' C, host float32) every
    element of it is checked against the same oracle rows, outside the timed
    part (each block of rows is timed on its own)."""
    import numpy as np
    import oracle
    from fp32_gemm_tile_amd import workloads as wl

    A, B, C = wl.make_inputs(w)
    threads = oracle.num_threads()
    oracle_s = 0.0
    worst, n_bad, err2, ref2 = 0.0, 0, 0.0, 0.0
    for r0 in range(0, w.M, block):
        rows = np.arange(r0, min(w.M, r0 + block), dtype=np.int64)
        t0 = time.perf_counter()
        cref, s = oracle.gemm_rows(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A, w.LDA, B,
                                   w.LDB, w.beta, C, w.LDC, rows=rows)
        oracle_s += time.perf_counter() - t0
        if gpu_out is not None:
            cin = C[rows, :w.N] if (C is not None and w.beta != 0) else None
            _, info = oracle.compare.check(gpu_out[rows], cref, s, w.K, w.alpha, w.beta, cin,
                                           frob=True)
            worst = max(worst, info["max_err_over_tol"])
            n_bad += info["n_bad"]
            err2 += info["frob_abs"] ** 2
            ref2 += info["frob_ref"] ** 2
    out = {"value": w.flops / oracle_s / 1e12, "unit": "TFLOP/s", "cores": threads,
           "cpu_model": cpu_model(), "kind": "oracle",
           "sample": f"the whole product: all {w.M} rows of {w.name} "
                     f"({w.M}x{w.N}x{w.K} {w.transA}{w.transB}), binary64 oracle, "
                     f"{oracle_s:.1f} s",
           "single_thread_256cubed_s": oracle_single_thread_small()}
    if gpu_out is not None:
        out["parity"] = {"elements": int(w.M) * int(w.N), "outside_bound": n_bad,
                         "max_err_over_tol": worst,
                         "frob_rel": (err2 ** 0.5) / (ref2 ** 0.5) if ref2 > 0 else None,
                         "ok": n_bad == 0 and (ref2 == 0 or (err2 / ref2) ** 0.5 <= 1e-5)}
    return out


_ONE_THREAD_SNIPPET = """
import sys, time
sys.path.insert(0, sys.argv[1])
import oracle
from fp32_gemm_tile_amd import workloads as wl
w = wl.WORKLOADS["C1"]
A, B, C = wl.make_inputs(w)
t0 = time.perf_counter()
oracle.gemm(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A, w.LDA, B, w.LDB, w.beta, C, w.LDC)
print(time.perf_counter() - t0, oracle.num_threads())
"""


def oracle_single_thread_small():
    """Wall time of the whole 256^3 product on one host thread (the oracle in
    a child process with OMP_NUM_THREADS=1), or None."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, "-c", _ONE_THREAD_SNIPPET, ROOT], env=env,
                           capture_output=True, text=True, timeout=120)
        t, threads = r.stdout.split()
        return round(float(t), 4) if int(threads) == 1 else None
    except Exception:
        return None


def copy_probe(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size: it reads and writes
    nbytes each, the reference for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy_probe: {reps} copies of {nbytes} bytes", file=sys.stderr, flush=True)


def run_one(name, steps, warmup, with_cpu, config=-1, splitk=False, cold=False,
            sample_clock=False, epilogue=None, streamk=False, min_warm_s=0.0,
            keep_output=False, quant=None):
    from fp32_gemm_tile_amd import workloads as wl
    w = wl.WORKLOADS[name] if isinstance(name, str) else name
    g = time_gpu(w, steps, warmup, config, splitk, cold, sample_clock, epilogue, streamk,
                 min_warm_s, keep_output=(with_cpu or keep_output) and quant is None,
                 quant=quant)
    tflops = w.flops / (g["ms_per_launch"] * 1e-3) / 1e12
    gbs = w.compulsory_bytes / (g["ms_per_launch"] * 1e-3) / 1e9
    # The counter records are of plain calls (no split, no fused epilogue).
    plain = not splitk and not streamk and epilogue is None and quant is None
    traffic = load_traffic(name, g["config"]) if plain and isinstance(name, str) else None
    # Bound: the matrix core above the ridge point, HBM below it.
    hbm_bound = w.flops / w.compulsory_bytes < PEAK_FP32_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP32_TFLOPS, 4),
                "traffic": traffic}
    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(g["ms_per_launch"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"sgemm_{w.M}x{w.N}x{w.K}_{w.transA.lower()}{w.transB.lower()}",
                   "M": w.M, "N": w.N, "K": w.K, "transA": w.transA, "transB": w.transB,
                   "alpha": w.alpha, "beta": w.beta, "inputs": f"{w.dist} seed {w.seed}",
                   "kernel_config": g["config"], "splitk_slices": g["splits"]},
        "pct_of_fp32_peak": round(100 * tflops / PEAK_FP32_TFLOPS, 2),
        "ms_median": round(g["ms_median"], 4),
        "ms_min": round(g["ms_min"], 4),
        "tflops_at_median": round(w.flops / (g["ms_median"] * 1e-3) / 1e12, 3),
        "caches": "cold (512 MiB written before each call)" if cold else "warm",
        "epilogue": epilogue or "alpha/beta only",
        "quantised_output": quant,
        "gpu_clock_mhz_under_load": g["clock_mhz"],
        "hbm_gbs_compulsory": round(gbs, 1),
        "roofline": roof,
    }
    if keep_output:
        out["_output"] = g["output"]
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(w, g["output"])
    return out


def _splitk_arg(args):
    """False: fg_sgemm; True: fg_sgemm_splitk with a library-chosen split;
    an int > 0: that many splits."""
    if args.splitk is None:
        return False
    return True if args.splitk < 0 else args.splitk


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C5a")
    ap.add_argument("--config", type=int, default=-1, help="force a table entry")
    ap.add_argument("--suite", action="store_true",
                    help="one line per workload C1..C6 (no CPU baseline)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured MFMA-peak and HBM-read probes and the "
                         "clock sampling under load")
    ap.add_argument("--epilogue", choices=("none", "relu", "gelu", "silu"), default=None,
                    help="time fg_sgemm_fused with row/column scales and biases and this "
                         "activation")
    ap.add_argument("--quant", choices=("bf16", "int8_row"), default=None,
                    help="time fg_sgemm_quant: C plus a quantised copy Q in this format")
    ap.add_argument("--streamk", action="store_true",
                    help="time fg_sgemm_streamk (split tail round; workspace as the library "
                         "asks)")
    ap.add_argument("--cold", action="store_true",
                    help="write 512 MiB before every timed call (operands out of cache)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run a plain device copy of 1 GiB three times "
                         "(reference for scaling HBM traffic counters)")
    ap.add_argument("--calibrate", action="store_true",
                    help="time every table entry on every workload (one line each)")
    ap.add_argument("--no-extras", action="store_true",
                    help="with the default workload, skip the 4096^3 and row-block lines")
    ap.add_argument("--few-row-threads", type=int, default=0, choices=(0, 256, 512, 1024),
                    help="workgroup size of the few-row kernel, B stored K x N "
                         "(fg_set_few_row_threads; 0 = library default)")
    ap.add_argument("--group-m", type=int, default=0,
                    help="raster band height in tile rows (fg_set_raster; 0 = library default)")
    ap.add_argument("--xcd-remap", type=int, choices=(0, 1), default=1,
                    help="1: renumber workgroups so each XCD gets a contiguous run of tiles "
                         "(library default); 0: hardware round-robin order")
    ap.add_argument("--ops", choices=("NN", "NT", "TN", "TT"), default=None,
                    help="operand layouts instead of the workload's (square workloads with "
                         "dense leading dimensions only: the same buffers read in that layout)")
    ap.add_argument("--launch-floor", action="store_true",
                    help="time the library's smallest launch instead: C = 0 through fg_sgemm "
                         "with alpha = beta = 0 on the workload's C (one fill kernel)")
    ap.add_argument("--splitk", type=int, nargs="?", const=-1, default=None,
                    help="time fg_sgemm_splitk (256 MiB workspace) instead of fg_sgemm; "
                         "optional value = split count (default: library-chosen)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: runs on one GPU only (--gpus 1); "
              "multi-GPU sharding is not implemented", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import fp32_gemm_tile_amd as fg
    fg.load_library()
    if fg.fg_set_raster(args.group_m, args.xcd_remap) != fg.FG_OK or \
            fg.fg_set_few_row_threads(args.few_row_threads) != fg.FG_OK:
        print(f"bench.py: {fg.fg_last_error()}", file=sys.stderr)
        sys.exit(2)

    if args.launch_floor:
        print(json.dumps(launch_floor(args.workload, args.steps)), flush=True)
        return

    if args.suite or args.calibrate:
        ids = range(fg.fg_num_configs()) if args.calibrate else [args.config]
        from fp32_gemm_tile_amd import workloads as wl
        names = ("C1", "C2", "C3", "C4", "C5a", "C5b", "C6", "S8", "G1", "G1T", "G8", "G8T",
                 "G32")
        for name in names:
            for cid in ids:
                # The few-row kernel re-reads op(B) once per 8 rows of C: far
                # too slow to time on the large-M shapes.
                if cid >= 0 and fg.fg_get_config(cid)["kind"] == fg.FG_KIND_SKINNY \
                        and wl.WORKLOADS[name].M > 2048:
                    continue
                r = run_one(name, args.steps, args.warmup, False, cid, _splitk_arg(args),
                            epilogue=args.epilogue, streamk=args.streamk, min_warm_s=0.2,
                            quant=args.quant)
                print(json.dumps({"workload": name, "config": r["config"]["kernel_config"],
                                  "forced": cid, "splitk": _splitk_arg(args),
                                  "epilogue": args.epilogue, "streamk": args.streamk,
                                  "quant": args.quant,
                                  "tflops": r["value"],
                                  "ms": r["ms_per_step"], "pct": r["pct_of_fp32_peak"],
                                  "roofline": r["roofline"]}),
                      flush=True)
        return

    # The CPU baseline leg (the whole oracle, timed; every element of the
    # timed calls' result checked against it) runs last, after the GPU work.
    # Every shape is also warmed for at least 0.2 s before it is timed: a
    # short kernel's first few calls run before the clock has ramped up
    # (2048^3 reads about 12% slower after only the warm-up calls).
    with_cpu = not args.no_cpu
    target = args.workload
    if args.ops:
        import dataclasses
        from fp32_gemm_tile_amd import workloads as wl
        w0 = wl.WORKLOADS[args.workload]
        if not (w0.M == w0.N == w0.K and w0.lda is None and w0.ldb is None and w0.ldc is None):
            print("bench.py: --ops takes a square workload with dense leading dimensions",
                  file=sys.stderr)
            sys.exit(2)
        target = dataclasses.replace(w0, name=f"{w0.name}_{args.ops}", transA=args.ops[0],
                                     transB=args.ops[1])
    r = run_one(target, args.steps, args.warmup, False, args.config, _splitk_arg(args),
                args.cold, sample_clock=not args.no_probes, epilogue=args.epilogue,
                streamk=args.streamk, min_warm_s=0.2, keep_output=with_cpu, quant=args.quant)
    # The 4096^3 shape of the metric, and one GPU's row block of 8192^3 split
    # over eight GPUs, timed in the same run.
    if args.workload == "C5a" and not args.no_extras:
        r["also"] = {}
        for extra in ("C6", "S8"):
            r2 = run_one(extra, args.steps, args.warmup, False, args.config, cold=args.cold,
                         epilogue=args.epilogue, min_warm_s=0.2)
            r["also"][r2["config"]["workload"]] = {
                k: r2[k] for k in ("value", "unit", "ms_per_step", "ms_median", "ms_min",
                                   "pct_of_fp32_peak")}
            r["also"][r2["config"]["workload"]]["kernel_config"] = r2["config"]["kernel_config"]
    if not args.no_probes:
        mp = measured_peaks()
        mp["pct_of_measured_mfma"] = round(100 * r["value"] / mp["mfma_tflops"], 2)
        r["measured_peaks"] = mp
    if with_cpu:
        from fp32_gemm_tile_amd import workloads as wl
        r["cpu_baseline"] = cpu_baseline(target if args.ops else wl.WORKLOADS[args.workload],
                                         r.pop("_output", None))
        # every element of the timed calls' result against the oracle
        r["parity"] = r["cpu_baseline"].get("parity")
    if args.copy_probe:
        copy_probe()
    print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
