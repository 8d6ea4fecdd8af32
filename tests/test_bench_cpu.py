"""bench.py on the host: its one-GPU contract, the traffic-record keying and
the CPU baseline leg (the oracle on a bounded row sample). No GPU needed."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300,
                          env=dict(os.environ, **(env or {})))


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU" in r.stderr
    r = _run([], env={"WORLD_SIZE": "2"})
    assert r.returncode == 2


def test_no_gpu_fails_loudly():
    pytest.importorskip("torch")
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = _run(["--steps", "1", "--warmup", "0", "--no-cpu"])
    assert r.returncode == 1 and "no GPU" in r.stderr


def test_traffic_records_are_keyed_by_kernel_sources():
    for name in ("C5a", "C6", "G1", "G8"):
        path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
        rec = json.load(open(path))
        current = rec["kernel_source_sha"] == bench.kernel_source_sha(rec["kernel_config"])
        # a record taken on other kernel sources is reported as unmeasured
        want = rec["bytes_per_launch"] if current else None
        assert bench.load_traffic(name, rec["kernel_config"]) == want, name
        assert bench.load_traffic(name, "mfma_64x64x16_w2x2_s4") is None  # another entry
    assert bench.kernel_source_sha("mfma_x") != bench.kernel_source_sha("few_rows")
    assert bench.load_traffic("no_such_workload", "mfma_x") is None


def test_cpu_baseline_leg():
    """The oracle on the whole workload, timed; with a result given, every
    element is checked against it (an element off by far more than the bound
    is reported)."""
    import numpy as np
    import oracle
    from fp32_gemm_tile_amd import workloads as wl
    w = wl.WORKLOADS["C1"]
    A, B, C = wl.make_inputs(w)
    cref, _ = oracle.gemm(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A, w.LDA, B, w.LDB,
                          w.beta, C, w.LDC)
    good = cref.astype(np.float32)
    r = bench.cpu_baseline(w, good, block=100)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert r["cores"] >= 1 and "all 256 rows" in r["sample"]
    assert r["parity"]["ok"] and r["parity"]["elements"] == 256 * 256
    assert r["parity"]["outside_bound"] == 0 and r["parity"]["max_err_over_tol"] < 1
    bad = good.copy()
    bad[200, 17] += 1.0   # far above the bound (8 K 2^-24 S + 1e-6, about 0.01 here)
    r = bench.cpu_baseline(w, bad, block=64)
    assert not r["parity"]["ok"] and r["parity"]["outside_bound"] == 1
    t = r["single_thread_256cubed_s"]
    assert t is None or 0 < t < 60
    assert "parity" not in bench.cpu_baseline(w)
