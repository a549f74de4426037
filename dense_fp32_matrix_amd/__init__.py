"""Python binding of ``libsgemm.so``: row-major FP32 C = A.B, and the
library-call form C = alpha * op(A) op(B) + beta * C, on an MI355X.

Argument marshalling only -- every step of the product runs in the library's
gfx950 kernels.  The functions carry the C interface's names
(``include/sgemm.h``); tensors are torch CUDA (HIP) float32 matrices with unit
column stride, and the row stride is passed as the leading dimension.  If the
library has not been built, every call raises; there is no fallback.

SGEMM_LIBRARY, when set, names the library file to load instead of the
in-tree ``libsgemm.so`` -- used to run the same tests on the LDS-poison build
(``libsgemm_ldspoison.so``, see ``build.py``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "SgemmError", "PATHS", "DECOMPOSITIONS", "PACK", "TILE_ORDERS", "ROW_TAILS",
    "sgemm", "sgemm_ex", "sgemm_raw", "sgemm_plan_query", "sgemm_workspace_size",
    "gemm", "gemm_raw", "gemm_plan_query", "gemm_workspace_size", "gemm_noalloc", "gemm_noalloc_raw",
    "NOALLOC_SCRATCH_BYTES", "read_probe", "read_probe_raw", "READ_PROBE_PARTIALS",
    "fma_probe", "FMA_PROBE_FMAS_PER_ITER",
    "sgemm_tile_info", "sgemm_status_string", "sgemm_version", "library_path", "load_library",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("SGEMM_LIBRARY") or os.path.join(_HERE, "libsgemm.so")
_lib = None

PATHS = {"auto": 0, "naive": 1, "valu": 2, "mfma": 3, "skinny": 4}
_PATH_NAMES = {v: k for k, v in PATHS.items()}

SGEMM_OK = 0
_STATUS = {0: "SGEMM_OK", 1: "SGEMM_ERR_INVALID_ARG", 2: "SGEMM_ERR_UNSUPPORTED", 3: "SGEMM_ERR_HIP",
           4: "SGEMM_ERR_ALLOC", 5: "SGEMM_ERR_SCRATCH_LIMIT"}
NOALLOC_SCRATCH_BYTES = 128 << 20    # SGEMM_NOALLOC_SCRATCH_BYTES of the header


class SgemmError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {sgemm_status_string(status)}" if what else sgemm_status_string(status))


DECOMPOSITIONS = {"auto": 0, "tiles": 1, "stream_k": 2}
_DECOMP_NAMES = {v: k for k, v in DECOMPOSITIONS.items()}


class _Options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("tile", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("vector", ctypes.c_int32), ("decomposition", ctypes.c_int32), ("pack", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t), ("tile_order", ctypes.c_int32),
                ("row_tail", ctypes.c_int32)]


class _Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("tile", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("vector", ctypes.c_int32), ("bm", ctypes.c_int32), ("bn", ctypes.c_int32),
                ("bk", ctypes.c_int32), ("threads", ctypes.c_int32), ("tiles_m", ctypes.c_int64),
                ("tiles_n", ctypes.c_int64), ("k_chunk", ctypes.c_int64), ("workgroups", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t), ("launches", ctypes.c_int32),
                ("decomposition", ctypes.c_int32), ("dp_tiles", ctypes.c_int64), ("sk_tiles", ctypes.c_int64),
                ("sk_units_per_wg", ctypes.c_int64), ("packed", ctypes.c_int32), ("k_padded", ctypes.c_int32),
                ("tail_rows", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load ``libsgemm.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with dense_fp32_matrix_amd.build.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32
    mm = [i64, i64, i64, p, i64, p, i64, p, i64]
    lib.sgemm.argtypes = mm + [p]
    lib.sgemm.restype = ctypes.c_int
    lib.sgemm_ex.argtypes = mm + [p, ctypes.POINTER(_Options)]
    lib.sgemm_ex.restype = ctypes.c_int
    lib.sgemm_plan_query.argtypes = mm + [ctypes.POINTER(_Options), ctypes.POINTER(_Plan)]
    lib.sgemm_plan_query.restype = ctypes.c_int
    lib.sgemm_workspace_size.argtypes = [i64] * 6
    lib.sgemm_workspace_size.restype = ctypes.c_size_t
    f = ctypes.c_float
    gm = [i32, i32, i64, i64, i64, f, p, i64, p, i64, f, p, i64]
    lib.sgemm_gemm.argtypes = gm + [p]
    lib.sgemm_gemm.restype = ctypes.c_int
    lib.sgemm_gemm_ex.argtypes = gm + [p, ctypes.POINTER(_Options)]
    lib.sgemm_gemm_ex.restype = ctypes.c_int
    lib.sgemm_gemm_noalloc.argtypes = gm + [p, ctypes.POINTER(_Options)]
    lib.sgemm_gemm_noalloc.restype = ctypes.c_int
    lib.sgemm_gemm_plan_query.argtypes = gm + [ctypes.POINTER(_Options), ctypes.POINTER(_Plan)]
    lib.sgemm_gemm_plan_query.restype = ctypes.c_int
    lib.sgemm_gemm_workspace_size.argtypes = [i32, i32] + [i64] * 6
    lib.sgemm_gemm_workspace_size.restype = ctypes.c_size_t
    ip = ctypes.POINTER(i32)
    lib.sgemm_tile_info.argtypes = [i32, i32, ip, ip, ip, ip, ip]
    lib.sgemm_tile_info.restype = ctypes.c_int
    lib.sgemm_status_string.argtypes = [ctypes.c_int]
    lib.sgemm_status_string.restype = ctypes.c_char_p
    lib.sgemm_fma_probe.argtypes = [i32, i32, p, p]
    lib.sgemm_fma_probe.restype = ctypes.c_int
    lib.sgemm_read_probe.argtypes = [p, i64, p, p]
    lib.sgemm_read_probe.restype = ctypes.c_int
    lib.sgemm_version.argtypes = []
    lib.sgemm_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


PACK = {"auto": 0, "never": 1, "always": 2}


TILE_ORDERS = {"xcd": 0, "plain": 1}


ROW_TAILS = {"auto": 0, "never": 1, "always": 2}


def _options(path="auto", tile=-1, split_k=0, vector=0, decomposition="auto", workspace=None,
             workspace_bytes=0, pack="auto", tile_order="xcd", row_tail="auto") -> _Options:
    o = _Options()
    o.row_tail = ROW_TAILS[row_tail] if isinstance(row_tail, str) else int(row_tail)
    o.tile_order = TILE_ORDERS[tile_order] if isinstance(tile_order, str) else int(tile_order)
    o.pack = PACK[pack] if isinstance(pack, str) else int(pack)
    o.path = PATHS[path] if isinstance(path, str) else int(path)
    o.tile = int(tile)
    o.split_k = int(split_k)
    o.vector = int(vector)
    o.decomposition = DECOMPOSITIONS[decomposition] if isinstance(decomposition, str) else int(decomposition)
    if workspace is not None and not isinstance(workspace, int):
        workspace_bytes = workspace.numel() * workspace.element_size()
        workspace = workspace.data_ptr()
    o.workspace = workspace
    o.workspace_bytes = int(workspace_bytes)
    return o


def _check_tensor(t, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D torch tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be on a GPU")


def _storage_layout(shape, strides, name, allow_column_major=False):
    """(op, ld) of a 2-D view with this shape and these element strides:
    op 0 for a row-major view (ld = the row stride), op 1 for a column-major
    one (the transpose of a row-major matrix, ld = the column stride; only
    when allow_column_major).  Stored rows must not overlap: a leading
    dimension below the stored width -- a broadcast view with stride 0, or
    an as_strided view whose rows share elements -- is rejected rather than
    widened, which would address memory outside the tensor."""
    rows, cols = shape
    rs, cs = strides
    if cols <= 1 or cs == 1:
        if rows > 1 and rs < max(cols, 1):
            raise ValueError(f"{name}: row stride {rs} is below the row width {cols} (overlapping rows)")
        return 0, (rs if rows > 1 else max(cols, 1))
    if allow_column_major and (rows <= 1 or rs == 1):
        if cs < max(rows, 1):
            raise ValueError(f"{name}: column stride {cs} is below the column height {rows} (overlapping columns)")
        return 1, cs
    if allow_column_major:
        raise ValueError(f"{name} must be row-major or column-major (one unit stride)")
    raise ValueError(f"{name} must have unit column stride (row-major)")


def _matrix(t, name):
    """(pointer, rows, cols, ld) of a 2-D float32 row-major device tensor."""
    _check_tensor(t, name)
    rows, cols = t.shape
    _, ld = _storage_layout((rows, cols), t.stride(), name)
    return (t.data_ptr() if t.numel() else None), rows, cols, ld


def _stream_handle(stream, device):
    import torch
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def sgemm_raw(M, N, K, A, lda, B, ldb, C, ldc, stream=0, opts: Optional[_Options] = None) -> int:
    """The C call with integer device addresses; returns the status code."""
    lib = load_library()
    if opts is None:
        return lib.sgemm(M, N, K, A, lda, B, ldb, C, ldc, stream)
    return lib.sgemm_ex(M, N, K, A, lda, B, ldb, C, ldc, stream, ctypes.byref(opts))


def _call(A, B, C, stream, opts):
    import torch
    a, M, K, lda = _matrix(A, "A")
    b, K2, N, ldb = _matrix(B, "B")
    if K != K2:
        raise ValueError(f"inner dimensions differ: A is {M}x{K}, B is {K2}x{N}")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    c, Mc, Nc, ldc = _matrix(C, "C")
    if (Mc, Nc) != (M, N):
        raise ValueError(f"C must be {M}x{N}, got {Mc}x{Nc}")
    if not (A.device == B.device == C.device):
        raise ValueError("A, B and C must be on the same device")
    with torch.cuda.device(A.device):
        st = sgemm_raw(M, N, K, a, lda, b, ldb, c, ldc, _stream_handle(stream, A.device), opts)
    if st != SGEMM_OK:
        raise SgemmError(st, "sgemm")
    return C


def sgemm(A, B, C=None, stream=None):
    """C = A.B (overwrites and returns C; allocates it when None), enqueued on
    ``stream`` (default: torch's current stream of A's device)."""
    return _call(A, B, C, stream, None)


def sgemm_ex(A, B, C=None, stream=None, *, path="auto", tile=-1, split_k=0, vector=0, decomposition="auto",
             workspace=None, pack="auto", tile_order="xcd", row_tail="auto"):
    """``sgemm`` with explicit options: ``path`` in PATHS, ``tile`` index, ``split_k``
    slices, ``vector=1`` to force 4-byte loads, ``decomposition`` in DECOMPOSITIONS,
    ``pack`` in PACK (aligned copies of misaligned operands), optional ``workspace``
    tensor, ``tile_order`` in TILE_ORDERS, ``row_tail`` in ROW_TAILS."""
    return _call(A, B, C, stream, _options(path, tile, split_k, vector, decomposition, workspace, pack=pack,
                                           tile_order=tile_order, row_tail=row_tail))


def gemm_raw(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0,
             opts: Optional[_Options] = None) -> int:
    """sgemm_gemm / sgemm_gemm_ex with integer device addresses; returns the status code."""
    lib = load_library()
    if opts is None:
        return lib.sgemm_gemm(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
    return lib.sgemm_gemm_ex(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, ctypes.byref(opts))


def _operand(t, name):
    """(pointer, op, rows, cols, ld) of the logical 2-D operand t: a row-major
    tensor is passed as stored (op N); a column-major one (a transposed view of
    a row-major matrix) as the stored matrix with op T."""
    _check_tensor(t, name)
    rows, cols = t.shape
    op, ld = _storage_layout((rows, cols), t.stride(), name, allow_column_major=True)
    return (t.data_ptr() if t.numel() else None), op, rows, cols, ld


def gemm(A, B, C=None, stream=None, *, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, **options):
    """C = alpha * op(A) @ op(B) + beta * C with op(X) = X.T when trans_x.

    A and B may be row-major tensors or column-major views (such as W.t());
    each is handed to the library as stored, with the matching operation
    flag, so nothing is copied.  C (row-major) is read only when beta != 0
    and is allocated when None (then beta must be 0).  ``options`` are those
    of ``sgemm_ex``.  Returns C."""
    import torch
    a_log = A.t() if trans_a else A
    b_log = B.t() if trans_b else B
    a, op_a, M, K, lda = _operand(a_log, "A")
    b, op_b, K2, N, ldb = _operand(b_log, "B")
    if K != K2:
        raise ValueError(f"inner dimensions differ: op(A) is {M}x{K}, op(B) is {K2}x{N}")
    if C is None:
        if beta != 0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    c, Mc, Nc, ldc = _matrix(C, "C")
    if (Mc, Nc) != (M, N):
        raise ValueError(f"C must be {M}x{N}, got {Mc}x{Nc}")
    if not (A.device == B.device == C.device):
        raise ValueError("A, B and C must be on the same device")
    opts = _options(**options) if options else None
    with torch.cuda.device(A.device):
        st = gemm_raw(op_a, op_b, M, N, K, float(alpha), a, lda, b, ldb, float(beta), c, ldc,
                      _stream_handle(stream, A.device), opts)
    if st != SGEMM_OK:
        raise SgemmError(st, "sgemm_gemm")
    return C


READ_PROBE_PARTIALS = 4096


def read_probe_raw(x, n, partial, stream=0) -> int:
    """sgemm_read_probe with integer device addresses; returns the status code."""
    return load_library().sgemm_read_probe(x, n, partial, stream)


def read_probe(x, partial=None, stream=None):
    """Read the float32 tensor x (contiguous) once on the GPU: the read-rate
    probe.  Returns the READ_PROBE_PARTIALS per-workgroup sums."""
    import torch
    for t, name in ((x, "x"), (partial, "partial")):
        if t is not None and (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda
                              or not t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous float32 GPU tensor")
    if partial is None:
        partial = torch.empty(READ_PROBE_PARTIALS, dtype=torch.float32, device=x.device)
    if partial.numel() < READ_PROBE_PARTIALS or partial.device != x.device:
        raise ValueError(f"partial must hold {READ_PROBE_PARTIALS} floats on x's device")
    with torch.cuda.device(x.device):
        st = read_probe_raw(x.data_ptr() if x.numel() else None, x.numel(), partial.data_ptr(),
                            _stream_handle(stream, x.device))
    if st != SGEMM_OK:
        raise SgemmError(st, "sgemm_read_probe")
    return partial


FMA_PROBE_FMAS_PER_ITER = 128


def fma_probe(iters, workgroups, out=None, stream=None):
    """The FMA-rate probe on the current device: workgroups x 256 lanes, each
    FMA_PROBE_FMAS_PER_ITER x iters scalar FP32 FMAs.  Returns the per-lane
    results (workgroups x 256 floats)."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device())
    if out is None:
        out = torch.empty(int(workgroups) * 256, dtype=torch.float32, device=dev)
    if (out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous()
            or out.numel() < int(workgroups) * 256):
        raise ValueError("out must be a contiguous float32 GPU tensor of workgroups x 256 floats")
    with torch.cuda.device(out.device):
        st = load_library().sgemm_fma_probe(int(iters), int(workgroups), out.data_ptr(),
                                            _stream_handle(stream, out.device))
    if st != SGEMM_OK:
        raise SgemmError(st, "sgemm_fma_probe")
    return out


def gemm_noalloc_raw(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0,
                     opts: Optional[_Options] = None) -> int:
    """sgemm_gemm_noalloc with integer device addresses; returns the status code."""
    lib = load_library()
    return lib.sgemm_gemm_noalloc(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                                  ctypes.byref(opts) if opts is not None else None)


def gemm_noalloc(A, B, C, stream=None, *, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, **options):
    """``gemm`` through sgemm_gemm_noalloc: the library allocates no device
    memory for the call (its scratch is the static buffer of
    NOALLOC_SCRATCH_BYTES); C must be given.  ``options`` are those of
    ``sgemm_ex`` without a workspace."""
    a_log = A.t() if trans_a else A
    b_log = B.t() if trans_b else B
    a, op_a, M, K, lda = _operand(a_log, "A")
    b, op_b, K2, N, ldb = _operand(b_log, "B")
    if K != K2:
        raise ValueError(f"inner dimensions differ: op(A) is {M}x{K}, op(B) is {K2}x{N}")
    c, Mc, Nc, ldc = _matrix(C, "C")
    if (Mc, Nc) != (M, N):
        raise ValueError(f"C must be {M}x{N}, got {Mc}x{Nc}")
    if not (A.device == B.device == C.device):
        raise ValueError("A, B and C must be on the same device")
    opts = _options(**options) if options else None
    import torch
    with torch.cuda.device(A.device):
        st = gemm_noalloc_raw(op_a, op_b, M, N, K, float(alpha), a, lda, b, ldb, float(beta), c, ldc,
                              _stream_handle(stream, A.device), opts)
    if st != SGEMM_OK:
        raise SgemmError(st, "sgemm_gemm_noalloc")
    return C


def gemm_plan_query(op_a, op_b, M, N, K, alpha=1.0, A=0x100000, lda=None, B=0x200000000, ldb=None, beta=0.0,
                    C=0x400000000, ldc=None, **options) -> dict:
    """The plan sgemm_gemm_ex would use (host only); ops are "N"/"T" or 0/1."""
    lib = load_library()
    oa = {"N": 0, "T": 1}.get(op_a, op_a)
    ob = {"N": 0, "T": 1}.get(op_b, op_b)
    lda = max(M if oa == 1 else K, 1) if lda is None else lda
    ldb = max(K if ob == 1 else N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    o = _options(**options)
    pl = _Plan()
    st = lib.sgemm_gemm_plan_query(oa, ob, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ctypes.byref(o),
                                   ctypes.byref(pl))
    if st != SGEMM_OK:
        raise SgemmError(st, "sgemm_gemm_plan_query")
    out = {name: getattr(pl, name) for name, _ in _Plan._fields_}
    out["path_name"] = _PATH_NAMES.get(out["path"], "?")
    out["decomposition_name"] = _DECOMP_NAMES.get(out["decomposition"], "?")
    return out


def gemm_workspace_size(op_a, op_b, M, N, K, lda=None, ldb=None, ldc=None) -> int:
    lib = load_library()
    oa = {"N": 0, "T": 1}.get(op_a, op_a)
    ob = {"N": 0, "T": 1}.get(op_b, op_b)
    return int(lib.sgemm_gemm_workspace_size(oa, ob, M, N, K, max(M if oa == 1 else K, 1) if lda is None else lda,
                                             max(K if ob == 1 else N, 1) if ldb is None else ldb,
                                             max(N, 1) if ldc is None else ldc))


def sgemm_plan_query(M, N, K, A=0x100000, lda=None, B=0x200000000, ldb=None, C=0x400000000, ldc=None,
                     **options) -> dict:
    """The plan sgemm_ex would use for these sizes, leading dimensions and
    (integer) addresses.  Host only.  Raises SgemmError on invalid arguments."""
    lib = load_library()
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    o = _options(**options)
    pl = _Plan()
    st = lib.sgemm_plan_query(M, N, K, A, lda, B, ldb, C, ldc, ctypes.byref(o), ctypes.byref(pl))
    if st != SGEMM_OK:
        raise SgemmError(st, "sgemm_plan_query")
    out = {name: getattr(pl, name) for name, _ in _Plan._fields_}
    out["path_name"] = _PATH_NAMES.get(out["path"], "?")
    out["decomposition_name"] = _DECOMP_NAMES.get(out["decomposition"], "?")
    return out


def sgemm_workspace_size(M, N, K, lda=None, ldb=None, ldc=None) -> int:
    lib = load_library()
    return int(lib.sgemm_workspace_size(M, N, K, max(K, 1) if lda is None else lda,
                                        max(N, 1) if ldb is None else ldb, max(N, 1) if ldc is None else ldc))


def sgemm_tile_info(path, tile=0) -> Optional[dict]:
    lib = load_library()
    vals = [ctypes.c_int32() for _ in range(5)]
    p = PATHS[path] if isinstance(path, str) else int(path)
    st = lib.sgemm_tile_info(p, tile, *[ctypes.byref(v) for v in vals])
    if st != SGEMM_OK:
        return None
    count, bm, bn, bk, threads = (v.value for v in vals)
    return {"count": count, "bm": bm, "bn": bn, "bk": bk, "threads": threads}


def sgemm_status_string(status: int) -> str:
    try:
        return load_library().sgemm_status_string(status).decode()
    except RuntimeError:
        return _STATUS.get(status, f"status {status}")


def sgemm_version() -> str:
    return load_library().sgemm_version().decode()
