"""Fused epilogue on the GPU (fg_sgemm_fused) against the epilogue oracle:

    C = act(alpha * r_i * c_j * (op(A) op(B))_ij + beta * C_ij + u_i + w_j)

Float inputs: every element within oracle.compare.epilogue_tol. Integer
inputs with relu or no activation: every intermediate is exact in binary32,
so the result must equal the oracle's bit for bit, for every table entry.
"""
import numpy as np
import pytest

import fp32_gemm_tile_amd as fg
from fp32_gemm_tile_amd import workloads
import oracle
from oracle import compare
from oracle import epilogue as ep
from gpu_util import FullCheck, log, row_blocks, to_device

pytestmark = pytest.mark.gpu

ACTS = ("none", "relu", "gelu", "silu")


def _vectors(rng, M, N, kind="normal", which=(True, True, True, True)):
    if kind == "int":
        draw = lambda n, lo, hi: rng.integers(lo, hi + 1, n).astype(np.float32)
        vs = [draw(M, -3, 3), draw(N, -3, 3), draw(M, -20, 20), draw(N, -20, 20)]
    else:
        vs = [rng.uniform(0.5, 2.0, M).astype(np.float32) * rng.choice([-1, 1], M),
              rng.uniform(0.5, 2.0, N).astype(np.float32),
              rng.standard_normal(M).astype(np.float32),
              rng.standard_normal(N).astype(np.float32)]
    return [v if on else None for v, on in zip(vs, which)]


def run_fused(w, A, B, C, vecs, act, config=-1, c_fill=np.nan, full=False):
    """fg_sgemm_fused on host arrays; returns the M x N result (and, with
    full, the whole C buffer as read back)."""
    import torch
    dA, _ba = to_device(A)
    dB, _bb = to_device(B)
    if C is None:
        C = np.full((w.M, w.LDC), c_fill, dtype=np.float32)
    dC, _bc = to_device(C)
    keep = [to_device(v)[0] if v is not None else None for v in vecs]
    e = fg.make_epilogue(*[(t.data_ptr() if t is not None else 0) for t in keep], act)
    log(f"  fg_sgemm_fused {w.transA}{w.transB} M={w.M} N={w.N} K={w.K} alpha={w.alpha} "
        f"beta={w.beta} act={act} vecs={[v is not None for v in vecs]} cfg={config}")
    s = torch.cuda.current_stream()
    st = fg.fg_sgemm_fused(w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(), w.LDA,
                           dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC, e,
                           s.cuda_stream, config)
    if st != fg.FG_OK:
        raise fg.FgError(st, fg.fg_last_bad_arg(), fg.fg_last_error())
    s.synchronize()
    buf = dC.cpu().numpy().reshape(C.shape)
    return (buf[:, :w.N].copy(), buf) if full else buf[:, :w.N].copy()


def reference(w, A, B, C, vecs, act):
    s, S = oracle.gemm(w.transA, w.transB, w.M, w.N, w.K, 1.0, A, w.LDA, B, w.LDB, 0.0,
                       None, w.N)
    cin = C[:, :w.N] if (C is not None and w.beta != 0) else None
    d, v = ep.epilogue(s, w.alpha, w.beta, cin, *vecs, act=act)
    return d, v, S, cin


def check(w, A, B, C, vecs, act, out):
    d, v, S, cin = reference(w, A, B, C, vecs, act)
    ok, info = compare.check_epilogue(out, d, v, S, w.K, w.alpha, w.beta, cin, *vecs, act=act)
    assert ok, (w, act, info)
    return info


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("ops", ["NN", "NT", "TN", "TT"])
def test_fused_matches_oracle(act, ops):
    w = workloads.custom(300, 257, 129, ops[0], ops[1], alpha=1.5, beta=0.5, dist="normal",
                         seed=31)
    A, B, C = workloads.make_inputs(w)
    vecs = _vectors(np.random.default_rng(32), w.M, w.N)
    check(w, A, B, C, vecs, act, run_fused(w, A, B, C, vecs, act))


@pytest.mark.parametrize("which", [(True, False, False, False), (False, True, False, False),
                                   (False, False, True, False), (False, False, False, True),
                                   (False, False, False, False)])
def test_fused_each_vector_alone(which):
    w = workloads.custom(129, 200, 77, alpha=0.75, beta=0.0, dist="normal", seed=33)
    A, B, _ = workloads.make_inputs(w)
    vecs = _vectors(np.random.default_rng(34), w.M, w.N, which=which)
    check(w, A, B, None, vecs, "gelu", run_fused(w, A, B, None, vecs, "gelu"))


@pytest.mark.parametrize("config", range(fg.fg_num_configs()))
def test_fused_integer_exact_every_config(config):
    """Integer-valued operands, scales and biases: every partial result is an
    integer or half-integer far below 2^24, so the epilogue is exact in
    binary32 and the result equals the oracle's bit for bit."""
    for ops, act in (("NN", "relu"), ("TN", "none"), ("NT", "relu")):
        w = workloads.custom(200, 136, 70, ops[0], ops[1], alpha=2.0, beta=0.5, dist="int8",
                             seed=40 + config)
        A, B, C = workloads.make_inputs(w)
        vecs = _vectors(np.random.default_rng(50 + config), w.M, w.N, kind="int")
        out = run_fused(w, A, B, C, vecs, act, config=config)
        d, _, _, _ = reference(w, A, B, C, vecs, act)
        assert np.array_equal(out, d.astype(np.float32)), (config, ops, act)
    # Rows of C not 16-byte aligned (odd ldc; the matrix-core entries stage
    # the result through LDS there), ragged M and N; C's padding is a guard
    # band.
    for ops, act in (("NN", "relu"), ("TT", "none")):
        w = workloads.custom(97, 131, 45, ops[0], ops[1], alpha=-1.0, beta=2.0, dist="int8",
                             seed=60 + config, ldc=133)
        A, B, C = workloads.make_inputs(w)
        C[:, w.N:] = 2468.0
        vecs = _vectors(np.random.default_rng(61 + config), w.M, w.N, kind="int")
        out, buf = run_fused(w, A, B, C, vecs, act, config=config, full=True)
        d, _, _, _ = reference(w, A, B, C, vecs, act)
        assert np.array_equal(out, d.astype(np.float32)), (config, ops, act, "ldc 133")
        assert np.all(buf[:, w.N:] == 2468.0), (config, ops, act, "padding written")


@pytest.mark.parametrize("act", ["relu", "gelu"])
def test_fused_without_product(act):
    """K == 0 and alpha == 0 take the elementwise path: C = act(beta*C + u + w),
    also with beta == 1 (no quick return once an epilogue is asked for)."""
    rng = np.random.default_rng(60)
    for K, alpha, beta in ((0, 1.0, 1.0), (0, 1.0, 0.0), (64, 0.0, -2.0)):
        w = workloads.custom(37, 53, K, alpha=alpha, beta=beta, dist="normal", seed=61)
        A, B, C = workloads.make_inputs(w, with_c=True)
        vecs = _vectors(rng, w.M, w.N)
        out = run_fused(w, A, B, C, vecs, act)
        cin = C[:, :w.N].astype(np.float64)
        d, v = ep.epilogue(np.zeros((w.M, w.N)), alpha, beta, cin if beta != 0 else None,
                           *vecs, act=act)
        ok, info = compare.check_epilogue(out, d, v, np.zeros((w.M, w.N)), K, alpha, beta,
                                          cin, *vecs, act=act)
        assert ok, (K, alpha, beta, info)


def test_fused_beta_zero_ignores_nan_in_c():
    w = workloads.custom(70, 90, 40, dist="normal", seed=62)
    A, B, _ = workloads.make_inputs(w)
    vecs = _vectors(np.random.default_rng(63), w.M, w.N)
    out = run_fused(w, A, B, None, vecs, "silu", c_fill=np.nan)
    assert np.all(np.isfinite(out))
    check(w, A, B, None, vecs, "silu", out)


def test_fused_without_epilogue_equals_plain_call():
    import torch
    w = workloads.custom(333, 222, 111, "T", "N", alpha=1.25, beta=-0.5, dist="normal", seed=64)
    A, B, C = workloads.make_inputs(w)
    outs = []
    for fused in (False, True):
        dA, _a = to_device(A)
        dB, _b = to_device(B)
        dC, _c = to_device(C)
        args = (w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(), w.LDA,
                dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC)
        s = torch.cuda.current_stream().cuda_stream
        st = fg.fg_sgemm_fused(*args, None, s, -1) if fused else fg.fg_sgemm_ex(*args, s, -1)
        assert st == fg.FG_OK
        torch.cuda.synchronize()
        outs.append(dC.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_fused_large_full():
    """8192^3 NN with every vector and gelu, in the launch configuration the
    bench times, every element against the epilogue oracle (row blocks)."""
    w = workloads.WORKLOADS["C5a"]
    A, B, _ = workloads.make_inputs(w)
    vecs = _vectors(np.random.default_rng(65), w.M, w.N)
    out = run_fused(w, A, B, None, vecs, "gelu")
    assert np.all(np.isfinite(out))
    fc = FullCheck("fused 8192^3 gelu")
    for rows in row_blocks(w.M, 1024):
        s, S = oracle.gemm_rows(w.transA, w.transB, w.M, w.N, w.K, 1.0, A, w.LDA, B, w.LDB,
                                0.0, None, w.LDC, rows=rows)
        bv = [vecs[0][rows], vecs[1], vecs[2][rows], vecs[3]]
        d, v = ep.epilogue(s, w.alpha, w.beta, None, *bv, act="gelu")
        ok, info = compare.check_epilogue(out[rows], d, v, S, w.K, w.alpha, w.beta, None, *bv,
                                          act="gelu", frob=False)
        diff = out[rows].astype(np.float64) - d
        info["frob_abs"] = float(np.linalg.norm(diff))
        info["frob_ref"] = float(np.linalg.norm(d))
        fc.add(rows, info)
    fc.finish()


def test_torch_wrapper_fused():
    import torch
    g = torch.Generator().manual_seed(7)
    A = torch.randn(150, 70, generator=g).cuda()
    B = torch.randn(70, 90, generator=g).cuda()
    r = torch.rand(150, generator=g).cuda()
    wb = torch.randn(90, generator=g).cuda()
    C1 = torch.empty(150, 90, device="cuda")
    fg.sgemm(A, B, C1, alpha=0.5, row_scale=r, col_bias=wb, activation="silu")
    torch.cuda.synchronize()
    s, S = oracle.gemm("N", "N", 150, 90, 70, 1.0, A.cpu().numpy(), 70, B.cpu().numpy(), 90,
                       0.0, None, 90)
    vecs = [r.cpu().numpy(), None, None, wb.cpu().numpy()]
    d, v = ep.epilogue(s, 0.5, 0.0, None, *vecs, act="silu")
    ok, info = compare.check_epilogue(C1.cpu().numpy(), d, v, S, 70, 0.5, 0.0, None, *vecs,
                                      act="silu")
    assert ok, info
    with pytest.raises(ValueError):
        fg.sgemm(A, B, C1, row_scale=torch.ones(149, device="cuda"))


@pytest.mark.parametrize("kernel", [1, 2])
@pytest.mark.parametrize("ops", ["NN", "NT", "TN", "TT"])
def test_fused_few_row_kernels(kernel, ops):
    """The fused epilogue in each few-row kernel family (1 vector ALU, 2
    matrix cores), forced, on few-row shapes with integer operands: bit for
    bit against the oracle."""
    cfg = [c["id"] for c in fg.configs() if c["kind"] == fg.FG_KIND_SKINNY][0]
    assert fg.fg_set_few_row_kernel(kernel) == fg.FG_OK
    try:
        for i, (M, N, K) in enumerate([(1, 300, 513), (5, 257, 130), (8, 8200, 64),
                                       (20, 100, 700)]):
            for act in ("relu", "silu"):
                w = workloads.custom(M, N, K, ops[0], ops[1], alpha=-1.5, beta=0.5,
                                     dist="int8", seed=60 + i)
                A, B, C = workloads.make_inputs(w)
                vecs = _vectors(np.random.default_rng(70 + i), M, N, kind="int")
                out = run_fused(w, A, B, C, vecs, act, config=cfg)
                if act == "relu":
                    d, _, _, _ = reference(w, A, B, C, vecs, act)
                    assert np.array_equal(out, d.astype(np.float32)), (kernel, ops, M, N, K)
                else:
                    check(w, A, B, C, vecs, act, out)
    finally:
        assert fg.fg_set_few_row_kernel(0) == fg.FG_OK
