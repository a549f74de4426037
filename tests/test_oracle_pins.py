"""Pins of the host oracle to facts outside itself.

The oracle follows the plain definition C[i][j] = sum_k A[i][k] B[k][j]
("CUDA 算子优化：GEMM", section "矩阵乘法").  Each test below fixes it against
something that does not reuse its code: exact integer arithmetic, closed
forms, identity and permutation matrices, the transpose law (row-major
C = AB is column-major C^T = B^T A^T, "GEMM from naive to tiled", section
二.2), associativity, a correctly rounded sum (math.fsum) and a library
float64 product.  The last group plants mistakes in calls to the oracle and
checks that the pins catch each one.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads

INT_SHAPES = [(1, 1, 1), (2, 5, 3), (7, 11, 13), (64, 64, 64), (300, 200, 20), (33, 1, 70), (1, 45, 9)]


def ints(rows, cols, seed):
    return workloads.draw(rows, cols, "integer", seed).numpy()


def unif(rows, cols, seed):
    return workloads.draw(rows, cols, "uniform", seed).numpy()


# --- exact integer brute force -------------------------------------------------

@pytest.mark.parametrize("M,N,K", INT_SHAPES)
def test_integer_inputs_exact(oracle_mod, M, N, K):
    A = ints(M, K, 1)
    B = ints(K, N, 2)
    exact = A.astype(np.int64) @ B.astype(np.int64)          # exact integer matmul
    exact_abs = np.abs(A).astype(np.int64) @ np.abs(B).astype(np.int64)
    C, D = oracle_mod.sgemm(A, B, with_denominator=True)
    assert np.array_equal(C, exact.astype(np.float64))
    assert np.array_equal(D, exact_abs.astype(np.float64))
    # and the binary32 rounding is exact too (|C| <= 16 K < 2^24)
    assert np.array_equal(oracle_mod.round_to_f32(C), exact.astype(np.float32))


def test_integer_triple_loop_tiny(oracle_mod):
    """A pure-Python i-j-k triple loop over Python ints (arbitrary precision)."""
    M, N, K = 3, 4, 5
    A = ints(M, K, 11)
    B = ints(K, N, 12)
    C = oracle_mod.sgemm(A, B)
    for i in range(M):
        for j in range(N):
            s = 0
            for k in range(K):
                s += int(A[i, k]) * int(B[k, j])
            assert C[i, j] == s


@pytest.mark.parametrize("M,N,K", [(5, 7, 3), (64, 33, 17)])
def test_entries_match_integer_product(oracle_mod, M, N, K):
    A = ints(M, K, 3)
    B = ints(K, N, 4)
    exact = A.astype(np.int64) @ B.astype(np.int64)
    exact_abs = np.abs(A).astype(np.int64) @ np.abs(B).astype(np.int64)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    c, d = oracle_mod.sgemm_entries(A, B, rows.ravel(), cols.ravel())
    assert np.array_equal(c, exact.ravel().astype(np.float64))
    assert np.array_equal(d, exact_abs.ravel().astype(np.float64))


# --- identity and permutation matrices -----------------------------------------

@pytest.mark.parametrize("M,N,K", [(9, 13, 7), (64, 48, 80)])
def test_identity_and_permutation(oracle_mod, M, N, K):
    A = unif(M, K, 5)
    B = unif(K, N, 6)
    I_K = np.eye(K, dtype=np.float32)
    I_M = np.eye(M, dtype=np.float32)
    assert np.array_equal(oracle_mod.sgemm(A, I_K), A.astype(np.float64))
    assert np.array_equal(oracle_mod.sgemm(I_M, A), A.astype(np.float64))
    rng = np.random.default_rng(7)
    p_rows = rng.permutation(M)
    P = np.zeros((M, M), dtype=np.float32)
    P[np.arange(M), p_rows] = 1.0            # (P A)[i] = A[p_rows[i]]
    assert np.array_equal(oracle_mod.sgemm(P, A), A[p_rows].astype(np.float64))
    p_cols = rng.permutation(N)
    Q = np.zeros((N, N), dtype=np.float32)
    Q[p_cols, np.arange(N)] = 1.0            # (B Q)[:, j] = B[:, p_cols[j]]
    assert np.array_equal(oracle_mod.sgemm(B, Q), B[:, p_cols].astype(np.float64))


# --- transpose law ---------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(5, 3, 8), (37, 29, 61), (128, 96, 200)])
def test_transpose_law_bitwise(oracle_mod, M, N, K):
    """(AB)^T = B^T A^T: same products, same ascending-k order -> same bits."""
    A = unif(M, K, 8)
    B = unif(K, N, 9)
    C = oracle_mod.sgemm(A, B)
    Ct = oracle_mod.sgemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(C.T, Ct)


# --- associativity ------------------------------------------------------------------

def test_associativity_integer_exact(oracle_mod):
    M, N, K = 6, 5, 7
    A = ints(M, K, 13)
    B = ints(K, N, 14)
    x = ints(N, 1, 15)[:, 0]
    lhs = oracle_mod.sgemm(A, B) @ x.astype(np.float64)            # (AB) x
    Bx = oracle_mod.sgemm(B, x.reshape(N, 1)).ravel()              # B x through the oracle
    rhs = oracle_mod.sgemm(A, Bx.astype(np.float32).reshape(K, 1)).ravel()  # A (B x)
    assert np.array_equal(lhs, rhs)
    # and through the gemv helper
    assert np.array_equal(oracle_mod.gemv(A, oracle_mod.gemv(B, x.astype(np.float64))), lhs)


def test_associativity_float_bound(oracle_mod):
    M, N, K = 17, 23, 31
    A = unif(M, K, 16)
    B = unif(K, N, 17)
    x = unif(N, 1, 18)[:, 0].astype(np.float64)
    lhs = oracle_mod.sgemm(A, B) @ x
    rhs = oracle_mod.gemv(A, oracle_mod.gemv(B, x))
    scale = oracle_mod.gemv(A, oracle_mod.gemv(B, np.abs(x), absolute=True), absolute=True)
    assert np.all(np.abs(lhs - rhs) <= 1e-12 * scale)


@pytest.mark.parametrize("M,K", [(1, 1), (7, 13), (64, 300)])
def test_gemv_exact_integers(oracle_mod, M, K):
    """oracle.gemv, plain and with absolute values, against exact int64
    arithmetic: y = A x and |A| |x| (the error scale of the full-size
    associativity check), on a row-padded A whose gap holds NaN."""
    A = workloads.with_ld(workloads.draw(M, K, "integer", 41), K + 3).numpy()
    x = workloads.draw(K, 1, "integer", 42).numpy()[:, 0].astype(np.int64)
    Ai = np.asarray(A).astype(np.int64)
    y = oracle_mod.gemv(A, x.astype(np.float64))
    y_abs = oracle_mod.gemv(A, x.astype(np.float64), absolute=True)
    assert np.array_equal(y, (Ai @ x).astype(np.float64))
    assert np.array_equal(y_abs, (np.abs(Ai) @ np.abs(x)).astype(np.float64))


def test_gemv_absolute_is_a_bound(oracle_mod):
    """|A x| <= |A| |x| elementwise, with equality where A and x agree in sign;
    a mixed-sign case tells the absolute form from the plain one, so a flag
    that is ignored fails here."""
    A = np.array([[1.0, -2.0, 3.0], [-1.0, -1.0, -1.0]], dtype=np.float32)
    x = np.array([1.0, 1.0, -1.0])
    assert np.array_equal(oracle_mod.gemv(A, x), np.array([-4.0, -1.0]))
    assert np.array_equal(oracle_mod.gemv(A, x, absolute=True), np.array([6.0, 3.0]))
    U = unif(40, 50, 43)
    v = unif(50, 1, 44)[:, 0].astype(np.float64)
    assert np.all(np.abs(oracle_mod.gemv(U, v)) <= oracle_mod.gemv(U, v, absolute=True))
    P = np.abs(U)
    assert np.array_equal(oracle_mod.gemv(P, np.abs(v)), oracle_mod.gemv(U, v, absolute=True))


# --- closed forms -------------------------------------------------------------------

@pytest.mark.parametrize("K", [1, 2, 255, 4096, 5792])
def test_closed_form_ones_and_ramp(oracle_mod, K):
    M, N = 3, 4
    ones_A = np.ones((M, K), dtype=np.float32)
    ones_B = np.ones((K, N), dtype=np.float32)
    assert np.all(oracle_mod.sgemm(ones_A, ones_B) == K)
    ramp_B = np.repeat(np.arange(K, dtype=np.float32).reshape(K, 1), N, axis=1)  # B[k][j] = k
    assert np.all(oracle_mod.sgemm(ones_A, ramp_B) == K * (K - 1) // 2)


def test_closed_form_rank1_single_rounding(oracle_mod):
    """K = 1: C = u v^T; in fp64 the product is exact, and rounding it to fp32
    equals the correctly rounded binary32 product."""
    u = unif(50, 1, 19)
    v = unif(1, 40, 20)
    C = oracle_mod.sgemm(u, v)
    exact = u.astype(np.float64) * v.astype(np.float64)
    assert np.array_equal(C, exact)
    assert np.array_equal(oracle_mod.round_to_f32(C), u * v)   # numpy fp32 multiply, RNE


def test_round_to_f32_ties_to_even(oracle_mod):
    vals = np.array([1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, -(1 + 2.0 ** -24), 2.0 ** 24 + 1, 0.0, -0.0])
    want = np.array([1.0, 1 + 2.0 ** -22, -1.0, 2.0 ** 24, 0.0, -0.0], dtype=np.float32)
    got = oracle_mod.round_to_f32(vals)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


# --- within rounding of the exact sum ---------------------------------------------------

def test_close_to_correctly_rounded_sum(oracle_mod):
    """math.fsum returns the correctly rounded sum of exact fp64 products; the
    oracle's ascending fp64 sum is within (K-1) u_64 D of it."""
    M, N, K = 6, 7, 300
    A = unif(M, K, 21)
    B = unif(K, N, 22)
    C, D = oracle_mod.sgemm(A, B, with_denominator=True)
    u64 = Fraction(1, 2 ** 53)
    for i in range(M):
        for j in range(N):
            # fp32 x fp32 products are exact in fp64; sum them exactly as rationals
            prods = [Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)]
            exact = sum(prods, Fraction(0))
            exact_abs = sum((abs(p) for p in prods), Fraction(0))
            assert abs(Fraction(C[i, j]) - exact) <= (K - 1) * u64 * Fraction(D[i, j])
            assert abs(Fraction(D[i, j]) - exact_abs) <= (K - 1) * u64 * Fraction(D[i, j])
            assert C[i, j] == pytest.approx(math.fsum(float(p) for p in prods), rel=0, abs=K * 2.0 ** -53 * D[i, j])


def test_library_float64_cross_check(oracle_mod):
    M, N, K = 40, 30, 500
    A = unif(M, K, 23)
    B = unif(K, N, 24)
    C, D = oracle_mod.sgemm(A, B, with_denominator=True)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    assert np.all(np.abs(C - ref) <= 1e-13 * D)


def test_padded_leading_dimension(oracle_mod):
    """Views with row stride > width: the gap (NaN) is never read."""
    M, N, K = 19, 21, 23
    A = workloads.with_ld(workloads.draw(M, K, "integer", 25), K + 5).numpy()
    B = workloads.with_ld(workloads.draw(K, N, "integer", 26), N + 3).numpy()
    assert A.strides[0] == 4 * (K + 5)
    C = oracle_mod.sgemm(A, B)
    assert np.all(np.isfinite(C))
    assert np.array_equal(C, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64))
    rows = np.array([0, M - 1, 5]); cols = np.array([N - 1, 0, 7])
    c, _ = oracle_mod.sgemm_entries(A, B, rows, cols)
    assert np.array_equal(c, C[rows, cols])


def test_empty_and_degenerate(oracle_mod):
    A = np.zeros((4, 0), dtype=np.float32)
    B = np.zeros((0, 5), dtype=np.float32)
    C, D = oracle_mod.sgemm(A, B, with_denominator=True)    # empty sum
    assert C.shape == (4, 5) and np.all(C == 0) and np.all(D == 0)
    assert oracle_mod.sgemm(np.zeros((0, 3), np.float32), np.ones((3, 2), np.float32)).shape == (0, 2)
    assert oracle_mod.sgemm(np.ones((2, 3), np.float32), np.zeros((3, 0), np.float32)).shape == (2, 0)


def test_threads_do_not_change_results(oracle_mod):
    """Rows are independent: the same inputs give the same bits however the
    rows are split (compare a full call with row-by-row calls)."""
    M, N, K = 24, 17, 129
    A = unif(M, K, 27)
    B = unif(K, N, 28)
    C = oracle_mod.sgemm(A, B)
    for i in range(M):
        assert np.array_equal(oracle_mod.sgemm(A[i:i + 1], B)[0], C[i])
    # and with one thread or three
    n = oracle_mod.num_threads()
    try:
        for t in (1, 3):
            oracle_mod.set_num_threads(t)
            assert oracle_mod.num_threads() == t
            assert np.array_equal(oracle_mod.sgemm(A, B), C)
    finally:
        oracle_mod.set_num_threads(n)


# --- the library-call form: alpha * op(A) op(B) + beta * C ------------------------------

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True), (True, True)])
def test_gemm_worked_example(oracle_mod, ta, tb):
    """The hand-computed example of tests/golden/gemm_alpha_beta.json, with
    each operand stored as given or transposed."""
    import json
    g = json.load(open(__import__("os").path.join(GOLDEN, "gemm_alpha_beta.json")))
    A = np.array(g["A"], np.float32)
    B = np.array(g["B"], np.float32)
    C = np.array(g["C"], np.float32)
    As = np.ascontiguousarray(A.T) if ta else A
    Bs = np.ascontiguousarray(B.T) if tb else B
    got = oracle_mod.gemm(As, Bs, C, trans_a=ta, trans_b=tb, alpha=g["alpha"], beta=g["beta"])
    assert np.array_equal(got, np.array(g["expected"], np.float64))
    assert np.array_equal(oracle_mod.gemm(As, Bs, trans_a=ta, trans_b=tb), np.array(g["AB"], np.float64))


@pytest.mark.parametrize("M,N,K", [(7, 11, 13), (33, 1, 70), (1, 45, 9), (64, 40, 17)])
def test_gemm_integer_exact_all_layouts(oracle_mod, M, N, K):
    """Integer operands, every storage layout, alpha = 2 and beta = -0.5: the
    result is exact, so it must equal the int64 product scaled by hand."""
    A = ints(M, K, 41)
    B = ints(K, N, 42)
    C = ints(M, N, 43)
    ref = 2.0 * (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64) - 0.5 * C.astype(np.float64)
    for ta in (False, True):
        for tb in (False, True):
            As = np.ascontiguousarray(A.T) if ta else A
            Bs = np.ascontiguousarray(B.T) if tb else B
            got = oracle_mod.gemm(As, Bs, C, trans_a=ta, trans_b=tb, alpha=2.0, beta=-0.5)
            assert np.array_equal(got, ref), (ta, tb)


def test_gemm_row_column_major_law(oracle_mod):
    """Section 二.2 of "GEMM from naive to tiled": row-major C = AB is C^T = B^T A^T.
    gemm with both operands transposed, fed B as the first and A as the second
    stored matrix, returns C^T with the same sums in the same order."""
    A = unif(37, 29, 44)
    B = unif(29, 23, 45)
    C = oracle_mod.sgemm(A, B)
    Ct = oracle_mod.gemm(B, A, trans_a=True, trans_b=True)
    assert Ct.shape == (23, 37)
    assert np.array_equal(Ct, C.T)


def test_gemm_scalars_skip_reads(oracle_mod):
    """beta == 0 does not read C; alpha == 0 does not read A or B (NaN there
    must not reach the result)."""
    A = unif(9, 12, 46)
    B = unif(12, 5, 47)
    Cnan = np.full((9, 5), np.nan, np.float32)
    got = oracle_mod.gemm(A, B, Cnan, alpha=3.0, beta=0.0)
    assert np.all(np.isfinite(got)) and np.array_equal(got, 3.0 * oracle_mod.sgemm(A, B))
    C = unif(9, 5, 48)
    got = oracle_mod.gemm(np.full_like(A, np.nan), np.full_like(B, np.nan), C, alpha=0.0, beta=-2.0)
    assert np.array_equal(got, -2.0 * C.astype(np.float64))
    got, D = oracle_mod.gemm(A, B, C, alpha=0.0, beta=0.0, with_denominator=True)
    assert np.all(got == 0) and np.all(D == 0)


def test_gemm_denominator(oracle_mod):
    """D = |alpha| |op(A)| |op(B)| + |beta| |C| on a case computed by hand."""
    A = np.array([[1, -2]], np.float32)
    B = np.array([[3], [4]], np.float32)
    C = np.array([[-5]], np.float32)
    val, D = oracle_mod.gemm(A, B, C, alpha=-2.0, beta=3.0, with_denominator=True)
    assert val[0, 0] == -2.0 * (3 - 8) + 3.0 * -5      # = -5
    assert D[0, 0] == 2.0 * (3 + 8) + 3.0 * 5           # = 37


# --- planted mistakes: each pin above must catch a plausible oracle bug ----------------

def _mutants(oracle_mod):
    def dropped_last_term(A, B):
        return oracle_mod.sgemm(np.ascontiguousarray(A[:, :-1]), np.ascontiguousarray(B[:-1, :]))

    def dropped_first_term(A, B):
        return oracle_mod.sgemm(np.ascontiguousarray(A[:, 1:]), np.ascontiguousarray(B[1:, :]))

    def transposed_b(A, B):
        return oracle_mod.sgemm(A, np.ascontiguousarray(B.T))

    def swapped_operands(A, B):
        return oracle_mod.sgemm(B, A)

    def flipped_sign(A, B):
        C = oracle_mod.sgemm(A, B)
        C[0, 0] = -C[0, 0]
        return C

    def off_by_one_row(A, B):
        return oracle_mod.sgemm(np.ascontiguousarray(np.roll(A, 1, axis=0)), B)

    return [dropped_last_term, dropped_first_term, transposed_b, swapped_operands, flipped_sign,
            off_by_one_row]


def test_planted_mistakes_are_caught(oracle_mod):
    K = 8
    A = ints(K, K, 31)       # square so that transposed / swapped calls run
    B = ints(K, K, 32)
    A[0, :] = 1.0            # C[0, 0] = column sum of B[:, 0] ...
    B[:, 0] = 1.0            # ... = K, nonzero, so the sign mutant shows
    exact = (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64)
    assert exact[0, 0] == K
    for mutant in _mutants(oracle_mod):
        got = mutant(A, B)
        assert not np.array_equal(got, exact), mutant.__name__


def test_planted_gemm_mistakes_are_caught(oracle_mod):
    """Plausible mistakes in the library-call form (an operand read with the
    wrong orientation, a scalar ignored or misapplied) fail the exact pin."""
    M, N, K = 6, 5, 7
    A = ints(M, K, 51)
    B = ints(K, N, 52)
    C = ints(M, N, 53)
    exact = 2.0 * (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64) - 0.5 * C.astype(np.float64)
    Bsq = ints(K, K, 54)
    mutants = {
        "trans flag ignored on A": lambda: oracle_mod.gemm(np.ascontiguousarray(A.T).reshape(M, K), B, C,
                                                            alpha=2.0, beta=-0.5),
        "alpha dropped": lambda: oracle_mod.gemm(A, B, C, alpha=1.0, beta=-0.5),
        "beta sign": lambda: oracle_mod.gemm(A, B, C, alpha=2.0, beta=0.5),
        "beta term dropped": lambda: oracle_mod.gemm(A, B, C, alpha=2.0, beta=0.0),
        "C read transposed-ish": lambda: oracle_mod.gemm(A, B, np.ascontiguousarray(np.roll(C, 1, axis=1)),
                                                          alpha=2.0, beta=-0.5),
    }
    for name, f in mutants.items():
        assert not np.array_equal(f(), exact), name
    # a square case where reading B with the wrong orientation still runs
    Asq = ints(K, K, 55)
    ref = (Asq.astype(np.int64) @ Bsq.astype(np.int64)).astype(np.float64)
    assert not np.array_equal(oracle_mod.gemm(Asq, Bsq, trans_b=True), ref)
    assert np.array_equal(oracle_mod.gemm(Asq, np.ascontiguousarray(Bsq.T), trans_b=True), ref)
