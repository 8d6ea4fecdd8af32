"""fp32_gemm_tile_amd -- true-fp32 SGEMM for MI355X (gfx950) behind a C ABI.

    C = alpha * op(A) * op(B) + beta * C     (row-major, see include/fp32gemm.h)

This module is a thin ctypes binding over ``libfp32gemm.so``: it marshals
arguments and nothing else; every step of the product runs in the library's
HIP kernels. There is no fallback: if the library is missing or cannot load,
importing the binding's functions raises.

Entry points (same names as the C ABI):
  fg_sgemm(...), fg_sgemm_ex(...)      raw pointers and sizes
  fg_sgemm_splitk(...), fg_sgemm_splitk_workspace_size(M, N, S)
  fg_num_configs(), fg_get_config(i), fg_select_config(...)
  fg_last_bad_arg(), fg_last_error(), fg_status_string(s), fg_abi_version()
Convenience:
  sgemm(A, B, C, alpha, beta, transA, transB, config=-1, stream=None)
      for torch tensors on the GPU (PyTorch only supplies memory and stream).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp32gemm.so")

FG_OP_N, FG_OP_T = 0, 1
FG_OK, FG_ERR_INVALID_ARG, FG_ERR_HIP, FG_ERR_UNSUPPORTED = 0, 1, 2, 3
FG_KIND_MFMA, FG_KIND_VALU, FG_KIND_SKINNY = 1, 2, 3
FG_MAX_LD = 2097152


class FgError(RuntimeError):
    def __init__(self, status, bad_arg, message):
        self.status = status
        self.bad_arg = bad_arg
        super().__init__(f"{status_name(status)} (bad argument {bad_arg}): {message}")


class fg_config(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("wm", ctypes.c_int32), ("wn", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("mr", ctypes.c_int32),
                ("name", ctypes.c_char * 40)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["name"] = self.name.decode()
        return d


FG_ACT_NONE, FG_ACT_RELU, FG_ACT_GELU, FG_ACT_SILU = 0, 1, 2, 3
_ACTS = {"none": FG_ACT_NONE, "relu": FG_ACT_RELU, "gelu": FG_ACT_GELU, "silu": FG_ACT_SILU}


class fg_epilogue(ctypes.Structure):
    _fields_ = [("row_scale", ctypes.c_void_p), ("col_scale", ctypes.c_void_p),
                ("row_bias", ctypes.c_void_p), ("col_bias", ctypes.c_void_p),
                ("activation", ctypes.c_int32)]


FG_QUANT_NONE, FG_QUANT_BF16, FG_QUANT_INT8_ROW = 0, 1, 2
_QUANTS = {"none": FG_QUANT_NONE, "bf16": FG_QUANT_BF16, "int8_row": FG_QUANT_INT8_ROW}


class fg_quant(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("out", ctypes.c_void_p), ("ldq", ctypes.c_int64),
                ("row_factor", ctypes.c_void_p)]


def make_quant(kind, out, ldq, row_factor=0):
    """fg_quant from a format ("bf16", "int8_row" or an fg_quant_kind), the
    device address of Q, its leading dimension and (int8_row) the device
    address of the M row factors."""
    k = _QUANTS[kind] if isinstance(kind, str) else int(kind)
    return fg_quant(k, out or None, ldq, row_factor or None)


def activation_code(act) -> int:
    """fg_activation value of "none" / "relu" / "gelu" / "silu" (or an int)."""
    if isinstance(act, str):
        if act not in _ACTS:
            raise ValueError(f"unknown activation {act!r}")
        return _ACTS[act]
    return int(act)


def make_epilogue(row_scale=0, col_scale=0, row_bias=0, col_bias=0, activation="none"):
    """fg_epilogue from device addresses (0 = not used) and an activation."""
    return fg_epilogue(row_scale or None, col_scale or None, row_bias or None,
                       col_bias or None, activation_code(activation))


_lib = None


def load_library(path: str = LIB_PATH):
    """Load (once) and return the ctypes handle. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
            " (there is no non-HIP fallback)")
    # One HIP runtime per process: PyTorch ships its own libamdhip64 (same
    # SONAME as the system one). Importing torch first makes the dynamic
    # loader bind this library to that copy, so torch's streams and device
    # pointers are the ones the library's runtime knows.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    gemm_args = [i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, vp]
    lib.fg_sgemm.argtypes = gemm_args
    lib.fg_sgemm.restype = i32
    lib.fg_sgemm_ex.argtypes = gemm_args + [i32]
    lib.fg_sgemm_ex.restype = i32
    lib.fg_sgemm_splitk.argtypes = gemm_args[:13] + [i32, vp, ctypes.c_size_t, vp]
    lib.fg_sgemm_splitk.restype = i32
    lib.fg_sgemm_splitk_noalloc.argtypes = gemm_args[:13] + [i32, vp]
    lib.fg_sgemm_splitk_noalloc.restype = i32
    lib.fg_sgemm_splitk_noalloc_max_bytes.argtypes = []
    lib.fg_sgemm_splitk_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.fg_sgemm_splitk_workspace_size.argtypes = [i64, i64, i32]
    lib.fg_sgemm_splitk_workspace_size.restype = ctypes.c_size_t
    lib.fg_num_configs.argtypes = []
    lib.fg_num_configs.restype = i32
    lib.fg_get_config.argtypes = [i32, ctypes.POINTER(fg_config)]
    lib.fg_get_config.restype = i32
    lib.fg_select_config.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64,
                                     ctypes.POINTER(fg_config)]
    lib.fg_select_config.restype = i32
    lib.fg_select_config_quant.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64,
                                           i32, ctypes.POINTER(fg_config)]
    lib.fg_select_config_quant.restype = i32
    lib.fg_select_config_ex.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, f32, vp, i64,
                                        i32, ctypes.c_size_t, i32, ctypes.POINTER(fg_config),
                                        ctypes.POINTER(i32)]
    lib.fg_select_config_ex.restype = i32
    lib.fg_last_bad_arg.argtypes = []
    lib.fg_last_bad_arg.restype = i32
    lib.fg_last_error.argtypes = []
    lib.fg_last_error.restype = ctypes.c_char_p
    lib.fg_status_string.argtypes = [i32]
    lib.fg_status_string.restype = ctypes.c_char_p
    lib.fg_abi_version.argtypes = []
    lib.fg_abi_version.restype = i32
    lib.fg_sgemm_streamk.argtypes = gemm_args[:13] + [vp, ctypes.c_size_t, vp]
    lib.fg_sgemm_streamk.restype = i32
    lib.fg_sgemm_streamk_workspace_size.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64]
    lib.fg_sgemm_streamk_workspace_size.restype = ctypes.c_size_t
    lib.fg_sgemm_fused.argtypes = gemm_args[:13] + [ctypes.POINTER(fg_epilogue), vp, i32]
    lib.fg_sgemm_fused.restype = i32
    lib.fg_sgemm_quant.argtypes = gemm_args[:13] + [ctypes.POINTER(fg_epilogue),
                                                    ctypes.POINTER(fg_quant), vp, i32]
    lib.fg_sgemm_quant.restype = i32
    lib.fg_estimate_seconds.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.fg_estimate_seconds.restype = ctypes.c_double
    lib.fg_get_efficiency.argtypes = [i32, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_double)]
    lib.fg_get_efficiency.restype = i32
    lib.fg_set_efficiency.argtypes = [i32, ctypes.c_double, ctypes.c_double]
    lib.fg_set_efficiency.restype = i32
    lib.fg_set_raster.argtypes = [i32, i32]
    lib.fg_set_raster.restype = i32
    lib.fg_get_raster.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.fg_get_raster.restype = i32
    lib.fg_set_few_row_threads.argtypes = [i32]
    lib.fg_set_few_row_threads.restype = i32
    lib.fg_set_few_row_kernel.argtypes = [i32]
    lib.fg_set_few_row_kernel.restype = i32
    lib.fg_get_model_constant.argtypes = [i32, ctypes.POINTER(ctypes.c_double)]
    lib.fg_get_model_constant.restype = i32
    lib.fg_set_model_constant.argtypes = [i32, ctypes.c_double]
    lib.fg_set_model_constant.restype = i32
    lib.fg_set_streamk_policy.argtypes = [i32]
    lib.fg_set_streamk_policy.restype = i32
    lib.fg_probe_mfma.argtypes = [i32, i32, vp, vp]
    lib.fg_probe_mfma.restype = i32
    lib.fg_probe_mfma_flops.argtypes = [i32, i32]
    lib.fg_probe_mfma_flops.restype = ctypes.c_double
    lib.fg_probe_lds_dma.argtypes = [vp, i32, vp, vp]
    lib.fg_probe_lds_dma.restype = i32
    lib.fg_probe_read.argtypes = [vp, i64, i32, vp, vp]
    lib.fg_probe_read.restype = i32
    _lib = lib
    return lib


def _op(t) -> int:
    if t in (0, 1):
        return int(t)
    if isinstance(t, str) and t.upper() in ("N", "T"):
        return FG_OP_T if t.upper() == "T" else FG_OP_N
    return int(t)  # let the library reject out-of-domain values


def status_name(s: int) -> str:
    return load_library().fg_status_string(int(s)).decode()


def _raise_if(st: int):
    if st != FG_OK:
        lib = load_library()
        raise FgError(st, lib.fg_last_bad_arg(), lib.fg_last_error().decode())


# ---- C-ABI mirror ---------------------------------------------------------

def fg_sgemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0):
    """Raw call: A, B, C are device addresses (int), stream a hipStream_t (int)."""
    return load_library().fg_sgemm(_op(transA), _op(transB), M, N, K, alpha, A, lda,
                                   B, ldb, beta, C, ldc, stream or None)


def fg_sgemm_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0,
                config_id=-1):
    return load_library().fg_sgemm_ex(_op(transA), _op(transB), M, N, K, alpha, A, lda,
                                      B, ldb, beta, C, ldc, stream or None, config_id)


def fg_sgemm_splitk(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                    workspace, workspace_bytes, stream=0):
    """Raw split-K call (see include/fp32gemm.h); workspace is a device address."""
    return load_library().fg_sgemm_splitk(_op(transA), _op(transB), M, N, K, alpha, A, lda,
                                          B, ldb, beta, C, ldc, splits, workspace or None,
                                          workspace_bytes, stream or None)


def fg_sgemm_splitk_noalloc(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                            splits, stream=0):
    """Split-K with the library's own device-resident scratch (no workspace
    argument, nothing allocated); see include/fp32gemm.h."""
    return load_library().fg_sgemm_splitk_noalloc(_op(transA), _op(transB), M, N, K, alpha, A,
                                                  lda, B, ldb, beta, C, ldc, splits,
                                                  stream or None)


def fg_sgemm_splitk_noalloc_max_bytes() -> int:
    return load_library().fg_sgemm_splitk_noalloc_max_bytes()


def fg_sgemm_splitk_workspace_size(M, N, splits) -> int:
    return load_library().fg_sgemm_splitk_workspace_size(M, N, splits)


def fg_num_configs() -> int:
    return load_library().fg_num_configs()


def fg_get_config(i: int) -> dict:
    c = fg_config()
    _raise_if(load_library().fg_get_config(i, ctypes.byref(c)))
    return c.as_dict()


def fg_select_config(transA, transB, M, N, K, A=0, lda=None, B=0, ldb=None, C=0,
                     ldc=None, quant=None) -> dict:
    """The entry fg_sgemm would run (with quant, a format name or FG_QUANT_*
    code: the entry fg_sgemm_quant would run)."""
    ta, tb = _op(transA), _op(transB)
    lda = lda if lda is not None else max(1, K if ta == FG_OP_N else M)
    ldb = ldb if ldb is not None else max(1, N if tb == FG_OP_N else K)
    ldc = ldc if ldc is not None else max(1, N)
    c = fg_config()
    lib = load_library()
    if quant is None:
        _raise_if(lib.fg_select_config(ta, tb, M, N, K, A or None, lda, B or None, ldb,
                                       C or None, ldc, ctypes.byref(c)))
    else:
        kind = quant if isinstance(quant, int) else _QUANTS[quant]
        _raise_if(lib.fg_select_config_quant(ta, tb, M, N, K, A or None, lda, B or None, ldb,
                                             C or None, ldc, kind, ctypes.byref(c)))
    return c.as_dict()


def fg_select_config_ex(transA, transB, M, N, K, A=0, lda=None, B=0, ldb=None, beta=0.0, C=0,
                        ldc=None, splits=1, workspace_bytes=0, quant=None):
    """(entry, split-K slices) a call runs with config_id -1: fg_sgemm
    (splits=1), fg_sgemm_splitk (splits 0 = library choice bounded by
    workspace_bytes, or a count) or fg_sgemm_quant (quant, a format name or
    FG_QUANT_* code), with beta taken into account."""
    ta, tb = _op(transA), _op(transB)
    lda = lda if lda is not None else max(1, K if ta == FG_OP_N else M)
    ldb = ldb if ldb is not None else max(1, N if tb == FG_OP_N else K)
    ldc = ldc if ldc is not None else max(1, N)
    kind = 0 if quant is None else (quant if isinstance(quant, int) else _QUANTS[quant])
    c = fg_config()
    n = ctypes.c_int32(0)
    _raise_if(load_library().fg_select_config_ex(ta, tb, M, N, K, A or None, lda, B or None, ldb,
                                                 beta, C or None, ldc, splits, workspace_bytes,
                                                 kind, ctypes.byref(c), ctypes.byref(n)))
    return c.as_dict(), n.value


def fg_last_bad_arg() -> int:
    return load_library().fg_last_bad_arg()


def fg_last_error() -> str:
    return load_library().fg_last_error().decode()


def fg_status_string(s: int) -> str:
    return status_name(s)


def fg_abi_version() -> int:
    return load_library().fg_abi_version()


def fg_sgemm_streamk(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                     workspace, workspace_bytes, stream=0):
    """Raw call with the stream-K tail (device addresses as ints)."""
    return load_library().fg_sgemm_streamk(_op(transA), _op(transB), M, N, K, alpha, A, lda,
                                           B, ldb, beta, C, ldc, workspace or None,
                                           workspace_bytes, stream or None)


def fg_sgemm_streamk_workspace_size(transA, transB, M, N, K, A=0, lda=None, B=0,
                                    ldb=None) -> int:
    ta, tb = _op(transA), _op(transB)
    lda = lda if lda is not None else max(1, M if ta else K)
    ldb = ldb if ldb is not None else max(1, K if tb else N)
    return load_library().fg_sgemm_streamk_workspace_size(ta, tb, M, N, K, A or None, lda,
                                                          B or None, ldb)


def fg_sgemm_fused(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                   epilogue=None, stream=0, config=-1):
    """Raw call with a fused epilogue (an fg_epilogue, or None for none)."""
    ep = ctypes.byref(epilogue) if epilogue is not None else None
    return load_library().fg_sgemm_fused(_op(transA), _op(transB), M, N, K, alpha, A, lda,
                                         B, ldb, beta, C, ldc, ep, stream or None, config)


def fg_sgemm_quant(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                   epilogue=None, quant=None, stream=0, config=-1):
    """Raw call: the fused GEMM plus a quantised copy Q of C (an fg_quant, or
    None for none); see include/fp32gemm.h."""
    ep = ctypes.byref(epilogue) if epilogue is not None else None
    q = ctypes.byref(quant) if quant is not None else None
    return load_library().fg_sgemm_quant(_op(transA), _op(transB), M, N, K, alpha, A, lda,
                                         B, ldb, beta, C, ldc, ep, q, stream or None, config)


def fg_estimate_seconds(M, N, K, config_id, splits=1, beta_zero=True) -> float:
    """Cost-model estimate of one call with a given entry (fp32gemm_tune.h)."""
    return load_library().fg_estimate_seconds(M, N, K, config_id, splits, int(bool(beta_zero)))


def fg_get_efficiency(config_id):
    """(eff, eff1) of a matrix-core entry."""
    e, e1 = ctypes.c_double(), ctypes.c_double()
    _raise_if(load_library().fg_get_efficiency(config_id, ctypes.byref(e), ctypes.byref(e1)))
    return e.value, e1.value


def fg_set_efficiency(config_id, eff, eff1) -> int:
    return load_library().fg_set_efficiency(config_id, eff, eff1)


def fg_set_streamk_policy(policy) -> int:
    """0: split the stream-K tail when the model expects a gain; 1: always."""
    return load_library().fg_set_streamk_policy(policy)


def fg_set_raster(group_m, xcd_remap) -> int:
    """Raster order of the matrix-core kernels (fp32gemm_tune.h): band height
    in tile rows (0 = default) and the XCD renumbering (1 on, 0 off)."""
    return load_library().fg_set_raster(group_m, xcd_remap)


def fg_set_few_row_threads(threads) -> int:
    """Workgroup size of the few-row kernel, B stored K x N (fp32gemm_tune.h):
    0 = automatic, else 256, 512 or 1024."""
    return load_library().fg_set_few_row_threads(threads)


MODEL_CONSTANTS = ("launch", "store_bw", "store_exposed", "stream_bw", "split_bw", "few_fixed",
                   "few_mfma")   # fg_model_constant, in order


def fg_get_model_constant(which) -> float:
    """A constant of the cost model (index or name of MODEL_CONSTANTS)."""
    w = which if isinstance(which, int) else MODEL_CONSTANTS.index(which)
    v = ctypes.c_double()
    _raise_if(load_library().fg_get_model_constant(w, ctypes.byref(v)))
    return v.value


def fg_set_model_constant(which, value) -> int:
    w = which if isinstance(which, int) else MODEL_CONSTANTS.index(which)
    return load_library().fg_set_model_constant(w, value)


def fg_set_few_row_kernel(kernel):
    """Few-row kernel family: 0 automatic, 1 vector ALU, 2 matrix cores
    (include/fp32gemm_tune.h)."""
    return load_library().fg_set_few_row_kernel(kernel)


def fg_get_raster():
    """(group_m, xcd_remap) in use."""
    g, x = ctypes.c_int32(), ctypes.c_int32()
    _raise_if(load_library().fg_get_raster(ctypes.byref(g), ctypes.byref(x)))
    return g.value, x.value


def fg_probe_mfma(workgroups, iterations, out, stream=0) -> int:
    """MFMA-only loop (fp32gemm_probe.h); out: device pointer, workgroups*256 floats."""
    return load_library().fg_probe_mfma(workgroups, iterations, out or None, stream or None)


def fg_probe_mfma_flops(workgroups, iterations) -> float:
    return load_library().fg_probe_mfma_flops(workgroups, iterations)


def fg_probe_lds_dma(src, bytes_per_lane, out, stream=0) -> int:
    """One direct-to-LDS load with lanes reversed, LDS copied to out
    (fp32gemm_probe.h); src and out: 64 * bytes_per_lane / 4 floats."""
    return load_library().fg_probe_lds_dma(src or None, bytes_per_lane, out or None,
                                           stream or None)


def fg_probe_read(x, n, workgroups, out, stream=0) -> int:
    """Streaming read of n floats (fp32gemm_probe.h); out: workgroups*4 floats."""
    return load_library().fg_probe_read(x or None, n, workgroups, out or None, stream or None)


def configs() -> list:
    return [fg_get_config(i) for i in range(fg_num_configs())]


# ---- torch convenience ----------------------------------------------------

def _ld(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its rows")
    return t.stride(0) if t.size(0) > 1 else max(1, t.size(1))


def sgemm(A, B, C, alpha=1.0, beta=0.0, transA="N", transB="N", config=-1, stream=None,
          row_scale=None, col_scale=None, row_bias=None, col_bias=None, activation="none"):
    """C <- alpha * op(A) @ op(B) + beta * C for float32 GPU tensors (row-major,
    unit inner stride; leading dimensions are taken from the row strides).
    With any of row_scale / col_scale / row_bias / col_bias (contiguous float32
    GPU vectors of length M or N) or an activation ("relu", "gelu", "silu"),
    C <- act(alpha * r_i * c_j * (op(A) op(B))_ij + beta * C_ij + u_i + w_j)
    through fg_sgemm_fused. Returns C. Enqueued on ``stream`` (default:
    torch's current stream)."""
    import torch
    for name, t in (("A", A), ("B", B), ("C", C)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
    ta, tb = _op(transA), _op(transB)
    M, N = C.shape
    K = A.shape[1] if ta == FG_OP_N else A.shape[0]
    if (A.shape[0] if ta == FG_OP_N else A.shape[1]) != M:
        raise ValueError("op(A) rows != C rows")
    if (B.shape[0] if tb == FG_OP_N else B.shape[1]) != K:
        raise ValueError("op(B) rows != op(A) columns")
    if (B.shape[1] if tb == FG_OP_N else B.shape[0]) != N:
        raise ValueError("op(B) columns != C columns")
    vecs = []
    for name, v, n in (("row_scale", row_scale, M), ("col_scale", col_scale, N),
                       ("row_bias", row_bias, M), ("col_bias", col_bias, N)):
        if v is None:
            vecs.append(0)
            continue
        if v.dtype != torch.float32 or not v.is_cuda or not v.is_contiguous() or v.numel() != n:
            raise ValueError(f"{name} must be a contiguous float32 GPU vector of length {n}")
        vecs.append(v.data_ptr())
    if stream is None:
        stream = torch.cuda.current_stream(C.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if any(vecs) or activation_code(activation) != FG_ACT_NONE:
        st = fg_sgemm_fused(ta, tb, M, N, K, float(alpha), A.data_ptr(), _ld(A, "A"),
                            B.data_ptr(), _ld(B, "B"), float(beta), C.data_ptr(), _ld(C, "C"),
                            make_epilogue(*vecs, activation), stream, config)
    else:
        st = fg_sgemm_ex(ta, tb, M, N, K, float(alpha), A.data_ptr(), _ld(A, "A"),
                         B.data_ptr(), _ld(B, "B"), float(beta), C.data_ptr(), _ld(C, "C"),
                         stream, config)
    _raise_if(st)
    return C
