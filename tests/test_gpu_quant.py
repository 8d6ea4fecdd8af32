"""The quantised second output of the fused epilogue (fg_sgemm_quant) on the
GPU: C must pass the GEMM (or epilogue) oracle's bound as for the plain call,
and Q must equal the quantiser oracle applied to the GPU's own binary32 C, bit
for bit (the quantised code is decided on that binary32 value: the kernel's
precision). With integer-valued inputs C is exact, and Q equals the oracle's
codes of the exact C too."""
import numpy as np
import pytest

import fp32_gemm_tile_amd as fg
from fp32_gemm_tile_amd import workloads as wl
import oracle
from oracle import compare
from oracle import epilogue as ep
from oracle import quantize as oq
from gpu_util import check_full, check_full_blocked, log, to_device

pytestmark = pytest.mark.gpu

KINDS = ("bf16", "int8_row")
OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
ESIZE = {"bf16": 2, "int8_row": 1}
GUARD = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fg.load_library()
    yield
    torch.cuda.synchronize()


def quant_ids():
    """Table entries that write Q (the others are refused with quantised calls)."""
    return [c["id"] for c in fg.configs()
            if c["kind"] == fg.FG_KIND_SKINNY
            or (c["kind"] == fg.FG_KIND_MFMA and c["wm"] * c["wn"] // 64 <= 128)]


def no_quant_ids():
    return [c["id"] for c in fg.configs() if c["id"] not in quant_ids()]


def row_factors(cref, rng):
    """s_i = 127 / max_j |C_ij| times a factor in [0.8, 1.3]: most rows fill
    the int8 range, some saturate."""
    mx = np.max(np.abs(cref), axis=1)
    mx = np.where(mx > 0, mx, 1.0)
    return (127.0 / mx * rng.uniform(0.8, 1.3, mx.shape)).astype(np.float32)


def run_quant(w, A, B, C, kind, s=None, vecs=(None, None, None, None), act="none", config=-1,
              ldq=None, q_off=0):
    """fg_sgemm_quant on host arrays. Returns (C result M x N, Q codes M x N,
    whole Q buffer with its guard bytes as uint8)."""
    import torch
    ldq = ldq or w.N
    es = ESIZE[kind]
    dA, _a = to_device(A)
    dB, _b = to_device(B)
    Cbuf = C if C is not None else np.full((w.M, w.LDC), np.nan, dtype=np.float32)
    dC, _c = to_device(Cbuf)
    nbytes = (q_off + w.M * ldq) * es + 64
    qbuf = torch.full((nbytes,), GUARD, dtype=torch.uint8, device="cuda")
    qaddr = qbuf.data_ptr() + q_off * es
    keep = [to_device(v)[0] if v is not None else None for v in vecs]
    e = fg.make_epilogue(*[(t.data_ptr() if t is not None else 0) for t in keep], act)
    ds = to_device(s)[0] if s is not None else None
    q = fg.make_quant(kind, qaddr, ldq, ds.data_ptr() if ds is not None else 0)
    log(f"  fg_sgemm_quant {w.transA}{w.transB} M={w.M} N={w.N} K={w.K} {kind} ldq={ldq} "
        f"q_off={q_off} act={act} cfg={config}")
    stream = torch.cuda.current_stream()
    st = fg.fg_sgemm_quant(w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(), w.LDA,
                           dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC, e, q,
                           stream.cuda_stream, config)
    if st != fg.FG_OK:
        raise fg.FgError(st, fg.fg_last_bad_arg(), fg.fg_last_error())
    stream.synchronize()
    cout = dC.cpu().numpy().reshape(Cbuf.shape)[:, :w.N].copy()
    raw = qbuf.cpu().numpy()
    body = raw[q_off * es:(q_off + w.M * ldq) * es]
    dt = np.uint16 if kind == "bf16" else np.int8
    codes = body.view(dt).reshape(w.M, ldq)[:, :w.N].copy()
    return cout, codes, raw


def check_q(kind, cout, codes, s):
    want = oq.quantize(cout, kind, s)
    bad = np.argwhere(codes != want)
    assert bad.size == 0, (kind, bad[:5].tolist(),
                           [(float(cout[i, j]), int(codes[i, j]), int(want[i, j]))
                            for i, j in bad[:3]])


def check_guard(raw, w, ldq, kind, q_off):
    es = ESIZE[kind]
    assert np.all(raw[:q_off * es] == GUARD), "bytes before Q written"
    assert np.all(raw[(q_off + w.M * ldq) * es:] == GUARD), "bytes after Q written"
    body = raw[q_off * es:(q_off + w.M * ldq) * es].reshape(w.M, ldq * es)
    assert np.all(body[:, w.N * es:] == GUARD), "padding of Q rows written"


@pytest.mark.parametrize("cfg", quant_ids())
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("ta,tb", OPS)
def test_quant_every_entry(cfg, kind, ta, tb):
    """Every entry that writes Q, both formats, all layouts; ragged shapes;
    Q rows aligned (vector stores) and not (odd ldq, base one element off)."""
    rng = np.random.default_rng(cfg * 7 + len(kind))
    for i, (M, N, K, ldq_pad, q_off) in enumerate([(97, 131, 45, 3, 0), (200, 136, 72, 0, 0),
                                                   (129, 260, 33, 4, 1)]):
        w = wl.custom(M, N, K, ta, tb, alpha=1.25, beta=-0.5, dist="normal", seed=30 + i)
        A, B, C = wl.make_inputs(w)
        cref, _ = oracle.gemm(ta, tb, M, N, K, w.alpha, A, w.LDA, B, w.LDB, w.beta, C, w.LDC)
        s = row_factors(cref, rng) if kind == "int8_row" else None
        ldq = N + ldq_pad
        cout, codes, raw = run_quant(w, A, B, C, kind, s, config=cfg, ldq=ldq, q_off=q_off)
        check_full(w, A, B, C, cout)
        check_q(kind, cout, codes, s)
        check_guard(raw, w, ldq, kind, q_off)


@pytest.mark.parametrize("kind", KINDS)
def test_quant_integer_exact(kind):
    """Integer inputs: C is exact, so Q equals the oracle's codes of the exact
    result (not only of the GPU's C)."""
    rng = np.random.default_rng(3)
    for cfg in quant_ids():
        w = wl.custom(150, 90, 64, "N", "T", alpha=1.0, beta=2.0, dist="int8", seed=cfg)
        A, B, C = wl.make_inputs(w)
        cref, _ = oracle.gemm("N", "T", w.M, w.N, w.K, 1.0, A, w.LDA, B, w.LDB, 2.0, C, w.LDC)
        s = (rng.integers(1, 8, w.M) / 64.0).astype(np.float32) if kind == "int8_row" else None
        cout, codes, _ = run_quant(w, A, B, C, kind, s, config=cfg)
        assert np.array_equal(cout.astype(np.float64), cref), cfg
        assert np.array_equal(codes, oq.quantize(cref.astype(np.float32), kind, s)), cfg


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("act", ["none", "relu", "gelu", "silu"])
def test_quant_with_epilogue(kind, act):
    """Scales, biases and an activation before the quantiser (automatic entry)."""
    rng = np.random.default_rng(8)
    w = wl.custom(300, 257, 129, "T", "N", alpha=0.75, beta=0.5, dist="normal", seed=9)
    A, B, C = wl.make_inputs(w)
    vecs = [rng.uniform(0.5, 2.0, w.M).astype(np.float32),
            rng.uniform(0.5, 2.0, w.N).astype(np.float32),
            rng.standard_normal(w.M).astype(np.float32),
            rng.standard_normal(w.N).astype(np.float32)]
    s_, S = oracle.gemm(w.transA, w.transB, w.M, w.N, w.K, 1.0, A, w.LDA, B, w.LDB, 0.0,
                        None, w.N)
    d, v = ep.epilogue(s_, w.alpha, w.beta, C, *vecs, act=act)
    s = row_factors(d, rng) if kind == "int8_row" else None
    cout, codes, _ = run_quant(w, A, B, C, kind, s, vecs, act)
    ok, info = compare.check_epilogue(cout, d, v, S, w.K, w.alpha, w.beta, C, *vecs, act=act)
    assert ok, info
    check_q(kind, cout, codes, s)


@pytest.mark.parametrize("kind", KINDS)
def test_quant_nan_rows_and_saturation(kind):
    """A NaN in a row of A makes that row of C NaN: bf16 gives 0x7FC0, int8
    gives 0; a large factor saturates at -128 / 127."""
    w = wl.custom(64, 96, 40, dist="normal", seed=12)
    A, B, _ = wl.make_inputs(w)
    A[5, 7] = np.nan
    s = np.full(w.M, 1000.0, dtype=np.float32) if kind == "int8_row" else None
    cout, codes, _ = run_quant(w, A, B, None, kind, s)
    assert np.all(np.isnan(cout[5]))
    want_nan = 0x7FC0 if kind == "bf16" else 0
    assert np.all(codes[5].astype(np.int64) == want_nan)
    check_q(kind, cout, codes, s)
    if kind == "int8_row":
        assert np.any(codes == 127) and np.any(codes == -128)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("K,alpha,beta", [(0, 1.0, 0.5), (32, 0.0, -2.0), (0, 1.0, 1.0)])
def test_quant_scale_only_paths(kind, K, alpha, beta):
    """K == 0 or alpha == 0: C = beta * C (A and B unread), Q from it; with
    beta == 1 C is untouched but Q is still written."""
    M, N = 50, 70
    w = wl.custom(M, N, K, alpha=alpha, beta=beta, dist="normal", seed=13)
    A = np.full((M, max(K, 1)), np.nan, dtype=np.float32)
    B = np.full((max(K, 1), N), np.nan, dtype=np.float32)
    C = np.random.default_rng(1).standard_normal((M, N)).astype(np.float32)
    s = np.full(M, 40.0, dtype=np.float32) if kind == "int8_row" else None
    cout, codes, _ = run_quant(w, A, B, C.copy(), kind, s)
    want = C if beta == 1.0 else (beta * C.astype(np.float64)).astype(np.float32)
    assert np.array_equal(cout, want)
    check_q(kind, cout, codes, s)


@pytest.mark.parametrize("kind", KINDS)
def test_quant_few_rows(kind):
    """The few-row kernel (a handful of rows of C) writes Q too."""
    rng = np.random.default_rng(14)
    for M in (1, 3, 8):
        w = wl.custom(M, 4096, 4096, dist="uniform", seed=M)
        A, B, _ = wl.make_inputs(w)
        cref, _ = oracle.gemm("N", "N", M, 4096, 4096, 1.0, A, w.LDA, B, w.LDB, 0.0)
        s = row_factors(cref, rng) if kind == "int8_row" else None
        assert fg.fg_select_config("N", "N", M, 4096, 4096)["kind"] == fg.FG_KIND_SKINNY
        cout, codes, _ = run_quant(w, A, B, None, kind, s)
        check_full(w, A, B, None, cout)
        check_q(kind, cout, codes, s)


def test_quant_refused_where_not_built():
    """Entries that do not write Q are refused (argument 17) before any work;
    the automatic choice avoids them (4096^3 otherwise takes the 256 x 256
    tile)."""
    import torch
    A = torch.zeros(64 * 64, device="cuda")
    q = torch.zeros(64 * 64, dtype=torch.int16, device="cuda")
    quant = fg.make_quant("bf16", q.data_ptr(), 64)
    for cfg in no_quant_ids():
        st = fg.fg_sgemm_quant("N", "N", 64, 64, 64, 1.0, A.data_ptr(), 64, A.data_ptr(), 64,
                               0.0, A.data_ptr(), 64, None, quant,
                               torch.cuda.current_stream().cuda_stream, cfg)
        assert st == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 17, cfg
    assert len(no_quant_ids()) >= 1


@pytest.mark.parametrize("kind", KINDS)
def test_quant_large_full(kind):
    """4096^3 NN, automatic entry: every element of C against the oracle and
    every code of Q against the quantiser of the GPU's C."""
    rng = np.random.default_rng(15)
    w = wl.WORKLOADS["C6"]
    A, B, _ = wl.make_inputs(w)
    s = rng.uniform(1.0, 3.0, w.M).astype(np.float32) if kind == "int8_row" else None
    cout, codes, _ = run_quant(w, A, B, None, kind, s)
    check_full_blocked(w, A, B, None, cout, name=f"4096^3 with {kind} Q")
    check_q(kind, cout, codes, s)


@pytest.mark.parametrize("few_kernel", [1, 2])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("ta,tb", OPS)
def test_quant_few_row_kernels(few_kernel, kind, ta, tb):
    """Q from each few-row kernel family (1 vector ALU, 2 matrix cores),
    forced, in every layout, with the fused epilogue on: codes bit for bit
    against the oracle quantiser of the kernel's own C, C within the bound."""
    cfg = [c["id"] for c in fg.configs() if c["kind"] == fg.FG_KIND_SKINNY][0]
    rng = np.random.default_rng(80)
    assert fg.fg_set_few_row_kernel(few_kernel) == fg.FG_OK
    try:
        for M, N, K in [(1, 513, 700), (6, 300, 129), (24, 8200, 96)]:
            w = wl.custom(M, N, K, ta, tb, alpha=1.0, beta=0.0, dist="uniform", seed=M + N)
            A, B, _ = wl.make_inputs(w)
            cref, _ = oracle.gemm(ta, tb, M, N, K, 1.0, A, w.LDA, B, w.LDB, 0.0)
            s = row_factors(cref, rng) if kind == "int8_row" else None
            cout, codes, raw = run_quant(w, A, B, None, kind, s, config=cfg)
            check_full(w, A, B, None, cout)
            check_q(kind, cout, codes, s)
            check_guard(raw, w, w.N, kind, 0)
    finally:
        assert fg.fg_set_few_row_kernel(0) == fg.FG_OK
