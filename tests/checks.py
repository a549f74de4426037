"""Comparison helpers for the parity tests (test code; uses the oracle).

Acceptance bound: |C - C_ref| <= tol * D elementwise, with
D = sum_k |A_ik| |B_kj| and tol = 1e-5.  Where D = 0 the row of A or the
column of B is zero and C must be exactly zero.

Why 1e-5 (derivation, not a page figure): an FP32 sum of K products in any
order has error at most gamma_K * D with gamma_K ~ K u, u = 2^-24, and for
random-sign terms the typical error is ~u sqrt(K) sigma -- about 1e-7 D at the
configured sizes.  A dropped or repeated product of size |a b| ~ D / K moves
C by ~1/K of D, above 1e-5 for K <= ~65536 only for the larger terms, so the
integer-input tests (exact in any order) are the sharp check of indexing.
"""
import numpy as np

TOL = 1e-5


def normalized_error(C, Cref, D):
    """max over elements of |C - Cref| / D (D = 0 entries must match exactly)."""
    C = np.asarray(C, dtype=np.float64)
    err = np.abs(C - Cref)
    zero = D == 0
    if np.any(zero) and np.any(err[zero] != 0):
        return float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(zero, 0.0, err / np.where(zero, 1.0, D))
    return float(r.max()) if r.size else 0.0


def assert_within_bound(C, Cref, D, tol=TOL, what=""):
    C = np.asarray(C)
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"
    e = normalized_error(C, Cref, D)
    assert e <= tol, f"{what}: normalized error {e:.3e} > {tol:.0e}"
    return e


def assert_bit_exact(C, Cref32, what=""):
    C = np.asarray(C, dtype=np.float32)
    bad = np.flatnonzero(C.ravel() != Cref32.ravel())
    assert bad.size == 0, (f"{what}: {bad.size} elements differ; first at flat index {bad[0]}: "
                           f"{C.ravel()[bad[0]]} vs {Cref32.ravel()[bad[0]]}")
