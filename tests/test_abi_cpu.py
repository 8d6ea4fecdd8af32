"""The C-ABI library on the host: it loads, exports what the header declares,
validates arguments and takes the quick returns without touching a GPU.

Calls in this module pass made-up device addresses (16, 4096, ...). Every
call that could get past validation to a kernel launch runs in a child
process with the GPUs hidden (run_without_gpu), so even on a machine with a
GPU none of them can enqueue work on those addresses."""
import ctypes
import glob
import json
import os
import re
import subprocess
import sys

import pytest

import fp32_gemm_tile_amd as fg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp32gemm.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

# The statuses a call that passed validation may end with when no GPU is
# visible: it stops at the device check. FG_OK would mean work was enqueued.
NO_DEVICE = (fg.FG_ERR_HIP, fg.FG_ERR_UNSUPPORTED)

_HIDDEN_PRELUDE = f"""
import sys
sys.path.insert(0, {ROOT!r})
import torch
if torch.cuda.device_count() != 0:
    print("GPU-STILL-VISIBLE")
    sys.exit(0)
import fp32_gemm_tile_amd as fg
NO_DEVICE = (fg.FG_ERR_HIP, fg.FG_ERR_UNSUPPORTED)
"""


def run_without_gpu(code, timeout=300):
    """Run `code` in a child Python with every GPU hidden from the HIP runtime.
    The child checks first that torch sees no device and stops otherwise; the
    test is then skipped rather than risk a launch on made-up addresses."""
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", _HIDDEN_PRELUDE + code + "\nprint('ok')\n"],
                       env=env, capture_output=True, text=True, timeout=timeout)
    if "GPU-STILL-VISIBLE" in r.stdout:
        pytest.skip("could not hide the GPU from a child process")
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode,
                                                                   r.stderr[-1500:])


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(fg_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = fg.load_library()
    names = declared_functions()
    assert "fg_sgemm" in names and "fg_sgemm_ex" in names and "fg_probe_read" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"


def test_abi_version_and_status_strings():
    assert fg.fg_abi_version() == 2
    assert fg.fg_status_string(0) == "FG_OK"
    assert fg.fg_status_string(1) == "FG_ERR_INVALID_ARG"
    assert fg.fg_status_string(2) == "FG_ERR_HIP"
    assert fg.fg_status_string(3) == "FG_ERR_UNSUPPORTED"


def _call(ta=0, tb=0, M=4, N=4, K=4, alpha=1.0, A=16, lda=None, B=16, ldb=None,
          beta=0.0, C=16, ldc=None, cfg=-1):
    lda = lda if lda is not None else max(1, K if ta == 0 else M)
    ldb = ldb if ldb is not None else max(1, N if tb == 0 else K)
    ldc = ldc if ldc is not None else max(1, N)
    return fg.fg_sgemm_ex(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, 0, cfg)


@pytest.mark.parametrize("kw,bad", [
    (dict(ta=2), 1), (dict(tb=-1), 2), (dict(M=-1), 3), (dict(N=-1), 4), (dict(K=-1), 5),
    (dict(lda=3), 8), (dict(ta=1, M=6, lda=5), 8), (dict(ldb=3), 10),
    (dict(tb=1, K=7, ldb=6), 10), (dict(ldc=3), 13), (dict(A=0), 7), (dict(B=0), 9),
    (dict(C=0), 12), (dict(cfg=99), 15), (dict(cfg=-2), 15),
    (dict(M=0, lda=0), 8), (dict(N=0, ldc=0), 13),
])
def test_invalid_arguments_are_rejected_before_any_gpu_work(kw, bad):
    st = _call(**kw)
    assert st == fg.FG_ERR_INVALID_ARG
    assert fg.fg_last_bad_arg() == bad
    assert fg.fg_last_error()


@pytest.mark.parametrize("kw", [
    dict(M=0), dict(N=0), dict(M=0, N=0, K=0, C=0),
    dict(K=0, beta=1.0, A=0, B=0), dict(alpha=0.0, beta=1.0, A=0, B=0),
    dict(M=0, A=0, B=0, C=0),
])
def test_quick_returns_need_no_gpu(kw):
    # These must succeed without launching (there is no GPU here).
    assert _call(**kw) == fg.FG_OK
    assert fg.fg_last_bad_arg() == 0


def test_unsupported_leading_dimension():
    st = _call(lda=fg.FG_MAX_LD + 4)
    assert st == fg.FG_ERR_UNSUPPORTED


def test_config_table():
    n = fg.fg_num_configs()
    assert n >= 2
    cfgs = fg.configs()
    assert [c["id"] for c in cfgs] == list(range(n))
    kinds = {c["kind"] for c in cfgs}
    assert kinds == {fg.FG_KIND_MFMA, fg.FG_KIND_VALU, fg.FG_KIND_SKINNY}
    for c in cfgs:
        assert c["bm"] > 0 and c["bn"] > 0 and c["threads"] % 64 == 0
        assert c["bk"] > 0 or c["kind"] == fg.FG_KIND_SKINNY
        assert c["lds_bytes"] <= 160 * 1024
        if c["kind"] == fg.FG_KIND_MFMA:
            assert c["mr"] in (16, 32), c
            assert c["wm"] % c["mr"] == 0 and c["wn"] % c["mr"] == 0
            assert (c["bm"] // c["wm"]) * (c["bn"] // c["wn"]) * 64 == c["threads"]
    with pytest.raises(fg.FgError):
        fg.fg_get_config(n)


def test_few_rows_select_the_memory_bound_kernel():
    for M in (1, 2, 8):
        c = fg.fg_select_config("N", "N", M, 8192, 8192)
        assert c["kind"] == fg.FG_KIND_SKINNY, (M, c)
        c = fg.fg_select_config("N", "T", M, 8192, 8192)
        assert c["kind"] == fg.FG_KIND_SKINNY, (M, c)
    assert fg.fg_select_config("N", "N", 4096, 4096, 4096)["kind"] == fg.FG_KIND_MFMA


def test_selection_is_mfma_and_scales_with_shape():
    big = fg.fg_select_config("N", "N", 8192, 8192, 8192)
    assert big["kind"] == fg.FG_KIND_MFMA and big["bm"] * big["bn"] >= 256 * 128
    mid = fg.fg_select_config("N", "N", 2048, 2048, 2048)
    assert mid["kind"] == fg.FG_KIND_MFMA
    assert mid["bm"] * mid["bn"] < big["bm"] * big["bn"]
    # A few rows of C go to the few-row kernel; a grid that the large tiles
    # leave under-filled gets small MFMA tiles (measured on one MI355X:
    # 1024^3 takes 29 us with 64 x 64 tiles, 71 us with 128 x 128).
    for shape in ((1, 8192, 8192), (8, 4096, 4096), (32, 4096, 4096)):
        assert fg.fg_select_config("N", "N", *shape)["kind"] == fg.FG_KIND_SKINNY, shape
    small = fg.fg_select_config("N", "N", 1024, 1024, 1024)
    assert small["kind"] == fg.FG_KIND_MFMA and small["bm"] * small["bn"] <= 64 * 64
    ragged = fg.fg_select_config("T", "N", 3001, 2047, 1025, lda=3001, ldb=2047, ldc=2047)
    assert ragged["kind"] == fg.FG_KIND_MFMA
    # entries with 16-byte direct-to-LDS loads need 16-byte aligned rows of A
    # and B; unaligned calls get a 4-byte DMA entry (_dw) or a 2-stage one
    for c in (ragged, fg.fg_select_config("N", "N", 8192, 8192, 8192, A=16 + 4)):
        assert c["stages"] == 2 or "_dw" in c["name"], c
    with pytest.raises(fg.FgError) as e:
        fg.fg_select_config("N", "N", 4, 4, 4, lda=2)
    assert e.value.bad_arg == 8


def test_header_is_plain_c():
    """The headers compile as C99 with no HIP or torch headers."""
    import shutil
    import subprocess
    import tempfile
    if shutil.which("gcc") is None:
        pytest.skip("needs gcc")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        with open(src, "w") as f:
            f.write("".join(f'#include "{os.path.basename(h)}"\n' for h in HEADERS)
                    + "int main(void){return fg_abi_version()==0;}\n")
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                        "-I", os.path.dirname(HEADER), src], check=True)


def test_single_hip_runtime_in_process():
    """The library must bind to the HIP runtime torch already loaded (two
    runtimes in one process do not share streams)."""
    pytest.importorskip("torch")
    fg.load_library()
    maps = open("/proc/self/maps").read().splitlines()
    hip = {l.split()[-1] for l in maps if "libamdhip64" in l}
    assert len(hip) == 1, hip


def test_every_kernel_instance_is_linked():
    """Every kernel the launchers reference has its host launch stub in the
    library (clang once dropped some silently; the load then failed)."""
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("needs nm")
    out = subprocess.run(["nm", "-C", fg.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    undefined = [l for l in out.splitlines() if " U " in l and "device_stub" in l]
    assert not undefined, undefined[:5]
    assert sum(1 for l in out.splitlines() if "device_stub" in l and "sgemm_mfma" in l) >= 32


def test_auto_selection_matches_measured_best():
    """On every shape of the tile search (fp32_gemm_tile_amd/tuning/
    tile_search.json, timings of every searched instance on one MI355X), the
    entry the library picks runs within 2% of the fastest instance measured,
    and the kept table reaches the fastest within 1% (the cover's margin)."""
    from fp32_gemm_tile_amd import autotune
    rows, worst, geo = autotune.check_picks(autotune.REPORT_PATH, write_md=False)
    assert len(rows) >= 20
    bad = [r for r in rows if r["pick_over_best"] < 0.98]
    assert not bad, bad
    assert min(r["kept_over_best"] for r in rows) >= 0.99 - 1e-9
    assert geo > 0.99


def test_instance_list_matches_the_build():
    """Each matrix-core row of the table is a line of the instance list, and
    its waves per SIMD agree with the compiler's report of the last build
    (occupancy for its registers, capped by its LDS)."""
    from fp32_gemm_tile_amd import autotune, build
    entries = build.read_instances()
    mfma = [c for c in fg.configs() if c["kind"] == fg.FG_KIND_MFMA]
    assert [c["name"] for c in mfma] == [autotune.instance_name(e) for e in entries]
    assert [c["id"] for c in mfma] == list(range(len(entries)))
    if not glob.glob(os.path.join(build.BUILD, "sgemm_mfma_e*_00.resources.txt")):
        pytest.skip("no build report")
    for e in entries:
        assert autotune.occupancy(build.BUILD, e) == e["wps"], autotune.instance_name(e)
        if autotune.needs_aligned_rows(e):
            fb = entries[e["fallback"]]
            assert not autotune.needs_aligned_rows(fb), autotune.instance_name(e)


def test_splitk_workspace_size_and_validation():
    assert fg.fg_sgemm_splitk_workspace_size(100, 60, 1) == 0
    assert fg.fg_sgemm_splitk_workspace_size(100, 60, 0) == 0
    assert fg.fg_sgemm_splitk_workspace_size(0, 60, 4) == 0
    assert fg.fg_sgemm_splitk_workspace_size(100, 60, 4) == 100 * 60 * 4 * 4

    def call(splits=4, ws=4096, ws_bytes=1 << 30, M=64, N=64, K=1024):
        return fg.fg_sgemm_splitk(0, 0, M, N, K, 1.0, 16, K, 16, N, 0.0, 16, N, splits, ws,
                                  ws_bytes, 0)
    assert call(splits=-1) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 14
    assert call(ws=0) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 15
    assert call(ws=4098) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 15
    # 4 slices of 64 x 64 floats need 65536 bytes
    assert call(ws_bytes=65535) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 16
    # the usual argument checks still apply, with fg_sgemm's numbering
    assert fg.fg_sgemm_splitk(0, 0, 4, 4, 4, 1.0, 16, 3, 16, 4, 0.0, 16, 4, 2, 4096, 1 << 20,
                              0) == fg.FG_ERR_INVALID_ARG
    assert fg.fg_last_bad_arg() == 8
    # quick return: nothing to do, no GPU needed
    assert call(M=0) == fg.FG_OK


def test_splitk_auto_with_workspace_too_small_for_any_split():
    """splits = 0 with a workspace smaller than one M x N slice must plan a
    single pass (it once planned nothing and divided by zero). Without a GPU
    the call then stops at the device check."""
    run_without_gpu("""
st = fg.fg_sgemm_splitk(0, 0, 4096, 4096, 256, 1.0, 16, 256, 16, 4096, 0.0, 16, 4096, 0,
                        4096, 1024, 0)
assert st in NO_DEVICE, st
""")


@pytest.mark.parametrize("splits", [None, 0, 3])
def test_host_planner_handles_every_entry(splits):
    """Every table entry, forced, and split-K planning run through the host
    planner without crashing; with no GPU visible each call stops at the
    device check (FG_ERR_HIP or FG_ERR_UNSUPPORTED)."""
    run_without_gpu(f"""
for cid in range(fg.fg_num_configs()):
    for (M, N, K) in [(1, 1, 1), (8, 8192, 8192), (300, 257, 1025), (4096, 4096, 4096)]:
        st = fg.fg_sgemm_ex(0, 1, M, N, K, 1.0, 16, K, 16, K, 0.0, 16, N, 0, cid)
        assert st in NO_DEVICE, (cid, M, N, K, st)
for (M, N, K) in [(1, 1, 1), (8, 8192, 8192), (256, 256, 256), (300, 257, 1025)]:
    s = {splits!r}
    if s is None:
        st = fg.fg_sgemm(0, 0, M, N, K, 1.0, 16, K, 16, N, 0.5, 16, N, 0)
    else:
        st = fg.fg_sgemm_splitk(0, 0, M, N, K, 1.0, 16, K, 16, N, 0.5, 16, N, s, 4096, 1 << 30, 0)
    assert st in NO_DEVICE, (M, N, K, st)
""")


def test_probe_validation_and_flop_count():
    assert fg.fg_probe_mfma_flops(1024, 100) == 1024 * 4 * 100 * 4 * 4096
    assert fg.fg_probe_mfma_flops(0, 100) == 0.0
    assert fg.fg_probe_mfma(0, 10, 4096) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 1
    assert fg.fg_probe_mfma(4, 0, 4096) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 2
    assert fg.fg_probe_mfma(4, 10, 0) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 3
    assert fg.fg_probe_read(4096, 6, 4, 4096) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 2
    assert fg.fg_probe_read(4100, 8, 4, 4096) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 1
    assert fg.fg_probe_read(4096, 8, 0, 4096) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 3
    assert fg.fg_probe_read(4096, 8, 4, 0) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 4
    assert fg.fg_probe_lds_dma(0, 4, 4096) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 1
    assert fg.fg_probe_lds_dma(4096, 8, 4096) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 2
    assert fg.fg_probe_lds_dma(4096, 16, 0) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 3


def test_fused_validation_and_quick_returns():
    ep = fg.make_epilogue(activation="relu")
    call = lambda **kw: fg.fg_sgemm_fused(kw.get("ta", 0), 0, kw.get("M", 4), 4, kw.get("K", 4),
                                          kw.get("alpha", 1.0), 16, 4, 16, 4, kw.get("beta", 0.0),
                                          16, 4, kw.get("ep", ep), 0, kw.get("cfg", -1))
    bad = fg.make_epilogue(activation=7)
    assert call(ep=bad) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 14
    bad.activation = -1
    assert call(ep=bad) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 14
    assert call(cfg=fg.fg_num_configs()) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 16
    assert call(ta=5) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 1
    # nothing to do without a GPU: empty result
    assert call(M=0) == fg.FG_OK
    # K == 0 with beta == 1 is a no-op for the plain call, but not with an
    # activation: it must reach the device check (no GPU visible there)
    assert fg.fg_sgemm_fused(0, 0, 4, 4, 0, 1.0, 0, 1, 0, 4, 1.0, 16, 4, None, 0, -1) == fg.FG_OK
    run_without_gpu("""
ep = fg.make_epilogue(activation="relu")
st = fg.fg_sgemm_fused(0, 0, 4, 4, 0, 1.0, 16, 4, 16, 4, 1.0, 16, 4, ep, 0, -1)
assert st in NO_DEVICE and fg.fg_last_bad_arg() == 0, st
""")
    # an epilogue with nothing in it behaves as the plain call
    assert call(K=0, beta=1.0, ep=fg.make_epilogue()) == fg.FG_OK


def _id(name):
    return next(c["id"] for c in fg.configs() if c["name"] == name)


def _kind_id(kind):
    return next(c["id"] for c in fg.configs() if c["kind"] == kind)


def test_tuning_hooks():
    """The generated efficiency table is what the library uses, the model's
    estimate reacts to a changed efficiency, and the hooks validate."""
    import re
    inc = open(os.path.join(ROOT, "fp32_gemm_tile_amd", "csrc", "fg_tuned.inc")).read()
    rows = re.findall(r"\{(\d+|FG_ID_SKINNY), ([\d.]+), ([\d.]+)\}", inc)
    assert rows
    skinny, valu = _kind_id(fg.FG_KIND_SKINNY), _kind_id(fg.FG_KIND_VALU)
    for i, e, e1 in rows:
        got = fg.fg_get_efficiency(skinny if i == "FG_ID_SKINNY" else int(i))
        assert abs(got[0] - float(e)) < 1e-12 and abs(got[1] - float(e1)) < 1e-12
    big = _id("mfma_256x256x16_w2x2_s4")
    t0 = fg.fg_estimate_seconds(8192, 8192, 8192, big)
    # 2*8192^3 FLOP at the tuned efficiency, plus one launch and the tile
    # stores of four rounds (under 1% here)
    eff = fg.fg_get_efficiency(big)[0]
    assert abs(t0 / (2 * 8192 ** 3 / (eff * 157.3e12) + 3e-6) - 1) < 0.01
    old = fg.fg_get_efficiency(big)
    try:
        assert fg.fg_set_efficiency(big, old[0] / 2, old[1]) == fg.FG_OK
        assert abs(fg.fg_estimate_seconds(8192, 8192, 8192, big) / t0 - 2) < 0.02
    finally:
        assert fg.fg_set_efficiency(big, *old) == fg.FG_OK
    assert fg.fg_estimate_seconds(8192, 8192, 8192, valu) == -1.0   # vector-ALU entry
    assert fg.fg_estimate_seconds(1, 8192, 8192, skinny) > 0         # few-row entry
    assert fg.fg_set_efficiency(valu, 0.5, 0.5) == fg.FG_ERR_INVALID_ARG
    assert fg.fg_last_bad_arg() == 1
    assert fg.fg_set_efficiency(big, 0.0, 0.5) == fg.FG_ERR_INVALID_ARG
    assert fg.fg_last_bad_arg() == 2
    assert fg.fg_set_efficiency(big, 0.5, 1.5) == fg.FG_ERR_INVALID_ARG
    assert fg.fg_last_bad_arg() == 3
    with pytest.raises(fg.FgError):
        fg.fg_get_efficiency(valu)
    # the few-row entry has one efficiency dividing its modelled step time
    old_s = fg.fg_get_efficiency(skinny)
    t_s = fg.fg_estimate_seconds(64, 4096, 4096, skinny)
    try:
        fg.fg_set_efficiency(skinny, old_s[0] / 2, old_s[1])
        assert fg.fg_estimate_seconds(64, 4096, 4096, skinny) > 1.5 * t_s - 5e-6
    finally:
        fg.fg_set_efficiency(skinny, *old_s)


def test_autotune_fit_recovers_known_efficiencies():
    """The tuner's fit, given times that the model itself produces for known
    efficiencies, finds those efficiencies again (host only)."""
    from fp32_gemm_tile_amd import autotune
    # 64 x 64 tiles: several waves per SIMD, so both figures matter
    entry = _id("mfma_64x64x32_w2x2_s4_m16")
    old = fg.fg_get_efficiency(entry)
    shapes = [(256, 256, 256), (1024, 1024, 1024), (2048, 2048, 2048), (128, 4096, 4096),
              (4096, 4096, 4096)]
    try:
        fg.fg_set_efficiency(entry, 0.81, 0.47)
        samples = [(M, N, K, fg.fg_estimate_seconds(M, N, K, entry)) for M, N, K in shapes]
        eff, eff1, rms = autotune.fit_entry(entry, samples, True)
        assert (eff, eff1) == (0.81, 0.47) and rms < 1e-6
        assert fg.fg_get_efficiency(entry) == (0.81, 0.47)
    finally:
        fg.fg_set_efficiency(entry, *old)


def test_autotune_candidates():
    from fp32_gemm_tile_amd import autotune
    names = lambda sh: {fg.fg_get_config(i)["name"] for i in autotune.candidates(sh)}
    aligned = names((4096, 4096, 4096, "N", "N", None, None, None))
    ragged = names((3001, 2047, 1025, "T", "N", 3001, 2047, 2047))
    assert "mfma_256x256x16_w2x2_s4" in aligned and "few_rows" not in aligned
    assert "mfma_256x256x16_w2x2_s4" not in ragged
    assert ragged and all("_dw" in n for n in ragged), ragged
    assert "few_rows" in names((64, 4096, 4096, "N", "N", None, None, None))
    assert not any(n.startswith("valu_") and "skinny" not in n for n in aligned | ragged)


def test_search_space_respects_the_limits():
    """Every instance the search generates fits the LDS and the registers,
    splits its direct-to-LDS loads evenly over its waves, and its name is
    unique."""
    from fp32_gemm_tile_amd import autotune
    space = autotune.search_space()
    assert len(space) >= 40
    names = [autotune.instance_name(e) for e in space]
    assert len(set(names)) == len(names)
    for e in space:
        assert autotune.valid_instance(e), e
        assert e["stages"] * (e["bm"] + e["bn"]) * e["bk"] * 4 <= 160 * 1024
        acc, frag = autotune.registers(e)
        assert acc <= 256
    assert {e["bk"] for e in space} == {8, 16, 32} and {e["mr"] for e in space} == {16, 32}
    assert {e["dmab"] for e in space} == {4, 16}


def test_no_kernel_uses_scratch_memory():
    """Every kernel of the last build keeps its values in registers and LDS:
    the compiler's resource report (written by the build next to the
    objects) shows ScratchSize 0 for all of them. A spill of the
    accumulators once cost the matrix-core kernel its speed."""
    import re
    reports = glob.glob(os.path.join(ROOT, "_build", "*.resources.txt"))
    if not reports:
        pytest.skip("no build report (build with fp32_gemm_tile_amd/build.py)")
    sizes = []
    for path in reports:
        sizes += [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", open(path).read())]
    assert len(sizes) >= 40, len(sizes)
    assert max(sizes) == 0


def test_noalloc_limits_need_no_gpu():
    """fg_sgemm_splitk_noalloc refuses splits that do not fit its scratch
    before any device call; the limit is the one the header states."""
    cap = fg.fg_sgemm_splitk_noalloc_max_bytes()
    assert cap == 32 << 20
    call = lambda M, N, s: fg.fg_sgemm_splitk_noalloc(0, 0, M, N, 64, 1.0, 16, 64, 16, N, 0.0,
                                                      16, N, s, 0)
    assert call(2048, 2048, 3) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 14
    assert call(64, 64, -1) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 14
    assert call(0, 64, 4) == fg.FG_OK  # nothing to compute
    run_without_gpu("""
st = fg.fg_sgemm_splitk_noalloc(0, 0, 1024, 1024, 64, 1.0, 16, 64, 16, 1024, 0.0, 16, 1024, 8, 0)
assert st in NO_DEVICE, st
""")


def test_few_rows_entry_refuses_too_many_rows():
    """The few-row entry forced on more rows than its grid can hold: refused
    on the host (run with the GPU hidden, so nothing could launch anyway)."""
    run_without_gpu(f"""
few = [c["id"] for c in fg.configs() if c["kind"] == fg.FG_KIND_SKINNY][0]
st = fg.fg_sgemm_ex(0, 0, 65535 * 8 + 1, 4, 4, 1.0, 16, 4, 16, 4, 0.0, 16, 4, None, few)
assert st == fg.FG_ERR_UNSUPPORTED, st
assert "few-row entry" in fg.fg_last_error()
""")


def test_model_constants_hooks():
    """The cost model's shared constants: readable, settable within their
    domain (fractions at most 1), and they move the estimates."""
    assert len(fg.MODEL_CONSTANTS) == 7
    old = {c: fg.fg_get_model_constant(c) for c in fg.MODEL_CONSTANTS}
    assert all(v > 0 for v in old.values())
    big = [c["id"] for c in fg.configs() if c["name"] == "mfma_256x256x16_w2x2_s4"][0]
    few = [c["id"] for c in fg.configs() if c["kind"] == fg.FG_KIND_SKINNY][0]
    try:
        t = fg.fg_estimate_seconds(256, 256, 256, big)
        assert fg.fg_set_model_constant("launch", old["launch"] + 1e-3) == fg.FG_OK
        assert abs(fg.fg_estimate_seconds(256, 256, 256, big) - (t + 1e-3)) < 1e-9
        t = fg.fg_estimate_seconds(8, 8192, 8192, few)
        assert fg.fg_set_model_constant("stream_bw", old["stream_bw"] / 2) == fg.FG_OK
        assert fg.fg_estimate_seconds(8, 8192, 8192, few) > 1.5 * t - 1e-5
        for bad in (("store_exposed", 1.5), ("few_mfma", 0.0), ("launch", -1.0)):
            assert fg.fg_set_model_constant(*bad) == fg.FG_ERR_INVALID_ARG
            assert fg.fg_last_bad_arg() == 2
        assert fg.fg_set_model_constant(7, 1.0) == fg.FG_ERR_INVALID_ARG
        assert fg.fg_last_bad_arg() == 1
    finally:
        for c, v in old.items():
            assert fg.fg_set_model_constant(c, v) == fg.FG_OK


def test_select_config_quant_skips_entries_without_it():
    """The entry a quantised call runs: never one built without the quantised
    store; the same as the plain pick where that one has it."""
    quant_names = set()
    for kind in ("bf16", "int8_row"):
        for shape in [(8192, 8192, 8192), (4096, 4096, 4096), (3001, 2047, 1025), (1, 8192, 8192),
                      (256, 256, 256)]:
            plain = fg.fg_select_config("N", "N", *shape)
            q = fg.fg_select_config("N", "N", *shape, quant=kind)
            quant_names.add(q["name"])
            if plain["name"] != q["name"]:
                assert plain["kind"] == fg.FG_KIND_MFMA and plain["bm"] * plain["bn"] >= 256 * 256
    assert "mfma_256x256x16_w2x2_s4" not in quant_names
    with pytest.raises(fg.FgError):
        fg.fg_select_config("N", "N", 8, 8, 8, quant=7)


def test_select_config_ex_reports_what_the_call_runs():
    """fg_select_config_ex: with beta = 0, no split and no quantised output it
    is fg_select_config; a requested split runs on a matrix-core entry with
    that many slices (bounded by K); the library's own split stays inside the
    workspace; a workspace too small for a requested count is the call's own
    error (bad argument 14)."""
    shapes = [(8192, 8192, 8192), (4096, 4096, 4096), (3001, 2047, 1025), (1, 8192, 8192),
              (256, 256, 256), (2048, 2048, 2048), (16384, 16384, 256), (8, 8192, 8192)]
    for shape in shapes:
        for ta, tb in (("N", "N"), ("T", "N"), ("N", "T")):
            plain = fg.fg_select_config(ta, tb, *shape)
            assert fg.fg_select_config_ex(ta, tb, *shape) == (plain, 1)
            for kind in ("bf16", "int8_row"):
                q = fg.fg_select_config(ta, tb, *shape, quant=kind)
                assert fg.fg_select_config_ex(ta, tb, *shape, quant=kind) == (q, 1)
    ws = 1 << 28
    cfg, n = fg.fg_select_config_ex("N", "N", 256, 256, 256, splits=2, workspace_bytes=ws)
    assert cfg["kind"] == fg.FG_KIND_MFMA and n == 2
    # at most one slice per k-tile: K = 64 takes at most 64 / bk slices
    cfg, n = fg.fg_select_config_ex("N", "N", 256, 256, 64, splits=16, workspace_bytes=ws)
    assert n == 64 // cfg["bk"]
    cfg, n = fg.fg_select_config_ex("N", "N", 512, 512, 65536, splits=0, workspace_bytes=ws)
    assert n > 1 and n * 512 * 512 * 4 <= ws
    assert fg.fg_select_config_ex("N", "N", 512, 512, 65536, splits=0)[1] == 1  # no workspace
    with pytest.raises(fg.FgError) as e:
        fg.fg_select_config_ex("N", "N", 512, 512, 65536, splits=8, workspace_bytes=4 << 20)
    assert e.value.status == fg.FG_ERR_INVALID_ARG and e.value.bad_arg == 14
    lib = fg.load_library()
    c = fg.fg_config()
    n = ctypes.c_int32(0)
    call = lambda splits=1, kind=0, out=ctypes.byref(c): lib.fg_select_config_ex(
        0, 0, 64, 64, 64, None, 64, None, 64, 0.0, None, 64, splits, 0, kind, out,
        ctypes.byref(n))
    assert call() == fg.FG_OK
    assert call(splits=-1) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 13
    assert call(kind=9) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 15
    assert call(out=None) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 16


def test_quant_validation_needs_no_gpu():
    """fg_sgemm_quant checks its quantised-output description (argument 15)
    before any device work; an empty result needs nothing."""
    q = fg.make_quant("bf16", 4096, 4)
    call = lambda quant, M=4, N=4: fg.fg_sgemm_quant(0, 0, M, N, 4, 1.0, 16, 4, 16, N, 0.0, 16,
                                                     N, None, quant, 0, -1)
    assert call(fg.make_quant(7, 4096, 4)) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 15
    assert call(fg.make_quant("bf16", 4096, 3)) == fg.FG_ERR_INVALID_ARG
    assert fg.fg_last_bad_arg() == 15
    assert call(fg.make_quant("bf16", 0, 4)) == fg.FG_ERR_INVALID_ARG
    assert call(fg.make_quant("int8_row", 4096, 4, 0)) == fg.FG_ERR_INVALID_ARG
    assert fg.fg_last_bad_arg() == 15
    assert call(fg.make_quant("bf16", 4096, fg.FG_MAX_LD + 4)) == fg.FG_ERR_UNSUPPORTED
    assert call(q, M=0) == fg.FG_OK
    # a forced entry without the quantised store (the vector-ALU kernel) is
    # refused before the device check, as argument 17
    valu = next(c["id"] for c in fg.configs() if c["kind"] == fg.FG_KIND_VALU)
    st = fg.fg_sgemm_quant(0, 0, 4, 4, 4, 1.0, 16, 4, 16, 4, 0.0, 16, 4, None, q, 0, valu)
    assert st == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 17
    run_without_gpu("""
q = fg.make_quant("int8_row", 4096, 4, 8192)
st = fg.fg_sgemm_quant(0, 0, 4, 4, 0, 1.0, 16, 4, 16, 4, 1.0, 16, 4, None, q, 0, -1)
assert st in NO_DEVICE, st
""")


def test_raster_setting_validation():
    """fg_set_raster changes the tile order only through an explicit call;
    nothing in the environment does."""
    assert fg.fg_get_raster() == (0, 1)  # band height by layout, XCD renumbering on
    try:
        assert fg.fg_set_raster(-1, 1) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 1
        assert fg.fg_set_raster(4097, 1) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 1
        assert fg.fg_set_raster(4, 2) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 2
        assert fg.fg_set_raster(1, 0) == fg.FG_OK and fg.fg_get_raster() == (1, 0)
        assert fg.fg_set_raster(4, 1) == fg.FG_OK and fg.fg_get_raster() == (4, 1)
        assert fg.fg_set_raster(0, 1) == fg.FG_OK and fg.fg_get_raster() == (0, 1)
    finally:
        fg.fg_set_raster(0, 1)
    src = open(os.path.join(ROOT, "fp32_gemm_tile_amd", "csrc", "fg_api.cpp")).read()
    assert "getenv" not in src
    for t in (0, 256, 512, 1024):
        assert fg.fg_set_few_row_threads(t) == fg.FG_OK
    assert fg.fg_set_few_row_threads(128) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 1
    for k in (1, 2, 0):
        assert fg.fg_set_few_row_kernel(k) == fg.FG_OK
    assert fg.fg_set_few_row_kernel(3) == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 1
    fg.fg_set_few_row_threads(0)


def test_streamk_plan_and_validation():
    """Host side of fg_sgemm_streamk: the plan's workspace, the policy switch,
    argument checks (no GPU needed)."""
    try:
        assert fg.fg_set_streamk_policy(1) == fg.FG_OK
        need = fg.fg_sgemm_streamk_workspace_size("N", "N", 1000, 1000, 500)
        assert need > 0 and need % (64 * 64 * 4) == 0
        assert fg.fg_sgemm_streamk_workspace_size("N", "N", 8192, 8192, 8192) == 0  # no tail
        assert fg.fg_sgemm_streamk_workspace_size("N", "N", 4, 4, 0) == 0
        assert fg.fg_sgemm_streamk_workspace_size("N", "N", 4, 4, 4, lda=1) == 0    # invalid
        assert fg.fg_set_streamk_policy(0) == fg.FG_OK
        assert fg.fg_sgemm_streamk_workspace_size("N", "N", 1000, 1000, 500) <= need
        assert fg.fg_set_streamk_policy(2) == fg.FG_ERR_INVALID_ARG
    finally:
        fg.fg_set_streamk_policy(0)
    st = fg.fg_sgemm_streamk(0, 0, 64, 64, 64, 1.0, 16, 64, 16, 64, 0.0, 16, 64, 4100, 1 << 20, 0)
    assert st == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 14
    st = fg.fg_sgemm_streamk(0, 0, 64, 64, 64, 1.0, 16, 63, 16, 64, 0.0, 16, 64, 0, 0, 0)
    assert st == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 8
    assert fg.fg_sgemm_streamk(0, 0, 0, 64, 64, 1.0, 16, 64, 16, 64, 0.0, 16, 64, 0, 0, 0) == 0


def test_model_fit_runs_and_keeps_the_better_model(tmp_path):
    """autotune --fit-model on a copy of the search report, without sweeps:
    it reads the table's timings, compares the refitted model with the
    library as built, and writes nothing unless the refit is better."""
    import shutil
    from fp32_gemm_tile_amd import autotune
    rep = tmp_path / "report.json"
    shutil.copy(autotune.REPORT_PATH, rep)
    inc_before = open(autotune.INC_PATH).read()
    model_before = open(autotune.MODEL_INC).read()
    ids = [i for i in autotune.model_samples(json.load(open(rep)))]
    eff_before = {i: fg.fg_get_efficiency(i) for i in ids}
    const_before = {c: fg.fg_get_model_constant(c) for c in autotune.FIT_CONSTANTS}
    r = autotune.fit_model(str(rep), sweeps=0, write=False)
    assert r["samples"] >= 200
    assert r["before"]["geomean_pick"] > 0.99 and r["after"]["rms_log_error"] < 0.2
    assert open(autotune.INC_PATH).read() == inc_before
    assert open(autotune.MODEL_INC).read() == model_before
    if not r["written"]:
        # the loaded library's model is the one it was built with again
        assert {i: fg.fg_get_efficiency(i) for i in ids} == eff_before
        assert {c: fg.fg_get_model_constant(c) for c in autotune.FIT_CONSTANTS} == const_before
