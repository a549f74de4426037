"""Host reference SGEMM in fp64 -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and
the two share no code: the only common module is ``workloads`` (seeded
input generators, which hold none of the product's arithmetic).

Every function follows the plain definition C[i][j] = sum_k A[i][k] B[k][j]
("CUDA 算子优化：GEMM", section "矩阵乘法"; "GEMM from naive to tiled",
section 一.2) with fp64 accumulation in ascending k; ``gemm`` adds the
library-call form alpha * op(A) op(B) + beta * C ("GEMM from naive to
tiled", section 二.2).  Parity status: every
function here is pinned by ``tests/test_oracle_pins.py`` (integer brute
force, identity and permutation, transpose law, associativity, closed
forms, exact-sum and library cross-checks).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        lib.oracle_sgemm.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64]
        lib.oracle_sgemm.restype = ctypes.c_int
        lib.oracle_sgemm_entries.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64,
                                             _i64, _p, _p, _p, _p]
        lib.oracle_sgemm_entries.restype = ctypes.c_int
        lib.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, ctypes.c_double, _p, _i64,
                                    _p, _i64, ctypes.c_double, _p, _i64, _p, _i64, _p, _i64]
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_gemv.argtypes = [_i64, _i64, _p, _i64, _p, _p, ctypes.c_int]
        lib.oracle_gemv.restype = ctypes.c_int
        lib.oracle_round_to_f32.argtypes = [_i64, _p, _p]
        lib.oracle_round_to_f32.restype = None
        _lib = lib
    return _lib


def _as_matrix(x, name):
    """Row-major fp32 view (rows, cols) with unit column stride; returns (arr, ld)."""
    a = np.asarray(x)
    if a.dtype != np.float32 or a.ndim != 2:
        raise TypeError(f"{name}: need a 2-D float32 array, got {a.dtype} {a.shape}")
    if a.size == 0:
        return a, max(1, a.shape[1])
    if a.shape[1] > 1 and a.strides[1] != 4:
        raise ValueError(f"{name}: column stride must be 1 element")
    if a.shape[0] > 1 and a.strides[0] % 4:
        raise ValueError(f"{name}: row stride must be a whole number of elements")
    ld = a.strides[0] // 4 if a.shape[0] > 1 else max(1, a.shape[1])
    return a, ld


def _ptr(a):
    return a.ctypes.data if a.size else None


def num_threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the following calls (results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


def sgemm(A, B, with_denominator: bool = False):
    """C = A.B in fp64 (M x N), and optionally D = |A|.|B| (the error scale).

    A: (M, K) float32, B: (K, N) float32; row strides may exceed the width
    (a leading dimension with padding), column stride must be 1.
    """
    A, lda = _as_matrix(A, "A")
    B, ldb = _as_matrix(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    C = np.empty((M, N), dtype=np.float64)
    D = np.empty((M, N), dtype=np.float64) if with_denominator else None
    rc = _load().oracle_sgemm(M, N, K, _ptr(A), max(lda, K, 1), _ptr(B), max(ldb, N, 1),
                              _ptr(C), max(N, 1),
                              _ptr(D) if D is not None else None, max(N, 1))
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm failed ({rc})")
    return (C, D) if with_denominator else C


def gemm(A, B, C=None, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, with_denominator=False):
    """alpha * op(A) . op(B) + beta * C in fp64, and optionally its error scale.

    A is stored (M, K), or (K, M) when trans_a; B is stored (K, N), or (N, K)
    when trans_b (float32, unit column stride).  C (M, N) float32 is read
    only when beta != 0; A and B only when alpha != 0 and K > 0.  alpha and
    beta are taken as the float32 values a GPU call would receive.
    """
    A, lda = _as_matrix(A, "A")
    B, ldb = _as_matrix(B, "B")
    M, K = (A.shape[1], A.shape[0]) if trans_a else A.shape
    K2, N = (B.shape[1], B.shape[0]) if trans_b else B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    if beta != 0.0:
        if C is None:
            raise ValueError("beta != 0 needs C")
        C, ldcin = _as_matrix(C, "C")
        if C.shape != (M, N):
            raise ValueError(f"C must be {(M, N)}, got {C.shape}")
    else:
        C, ldcin = None, max(N, 1)
    out = np.empty((M, N), dtype=np.float64)
    D = np.empty((M, N), dtype=np.float64) if with_denominator else None
    rc = _load().oracle_gemm(int(bool(trans_a)), int(bool(trans_b)), M, N, K, alpha,
                             _ptr(A), max(lda, A.shape[1], 1), _ptr(B), max(ldb, B.shape[1], 1), beta,
                             _ptr(C) if C is not None else None, max(ldcin, N, 1),
                             _ptr(out), max(N, 1), _ptr(D) if D is not None else None, max(N, 1))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm failed ({rc})")
    return (out, D) if with_denominator else out


def sgemm_entries(A, B, rows, cols):
    """(C[rows[t], cols[t]], D[rows[t], cols[t]]) for each t, in fp64."""
    A, lda = _as_matrix(A, "A")
    B, ldb = _as_matrix(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    c = np.empty(rows.shape[0], dtype=np.float64)
    d = np.empty(rows.shape[0], dtype=np.float64)
    rc = _load().oracle_sgemm_entries(M, N, K, _ptr(A), max(lda, K, 1), _ptr(B), max(ldb, N, 1),
                                      rows.shape[0], _ptr(rows), _ptr(cols), _ptr(c), _ptr(d))
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm_entries failed ({rc})")
    return c, d


def gemv(A, x, absolute: bool = False):
    """y = A.x (or |A|.|x|) in fp64; A (M, K) float32, x length K."""
    A, lda = _as_matrix(A, "A")
    M, K = A.shape
    x = np.ascontiguousarray(x, dtype=np.float64)
    if x.shape != (K,):
        raise ValueError(f"x must have length {K}")
    y = np.empty(M, dtype=np.float64)
    rc = _load().oracle_gemv(M, K, _ptr(A), max(lda, K, 1), _ptr(x), _ptr(y), int(absolute))
    if rc != 0:
        raise RuntimeError(f"oracle_gemv failed ({rc})")
    return y


def round_to_f32(C):
    """fp64 -> binary32, round to nearest even."""
    C = np.ascontiguousarray(C, dtype=np.float64)
    out = np.empty(C.shape, dtype=np.float32)
    _load().oracle_round_to_f32(C.size, _ptr(C), _ptr(out))
    return out
