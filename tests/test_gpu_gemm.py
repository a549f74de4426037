"""GPU parity of the library-call form C = alpha * op(A) op(B) + beta * C
against the host oracle's ``gemm`` (the BLAS call that "GEMM from naive to
tiled", section 二.2, follows from torch.matmul; alpha and beta as in the
epilogue of section 九.2).

Bar (tests/checks.py): |C - C_ref| <= 1e-5 * D elementwise with
D = |alpha| sum_k |op(A)||op(B)| + |beta| |C_in|; bit-exact on small-integer
inputs with alpha = 2 and beta = -0.5, where every step is exact in FP32.
"""
import numpy as np
import pytest
import torch

import dense_fp32_matrix_amd as lib
import workloads
from checks import assert_bit_exact, assert_within_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def say(msg):
    print(f"[case] {msg}", flush=True)


def stored(M, N, K, ta, tb, kind, seed):
    """Stored operands (A is K x M when ta, B is N x K when tb) and C_in."""
    A = workloads.draw(K, M, kind, seed) if ta else workloads.draw(M, K, kind, seed)
    B = workloads.draw(N, K, kind, seed + 1) if tb else workloads.draw(K, N, kind, seed + 1)
    C = workloads.draw(M, N, kind, seed + 2)
    return A, B, C


def run_gemm(A, B, C, ta, tb, alpha, beta, **opts):
    Ad, Bd = A.to(DEV), B.to(DEV)
    Cd = C.to(DEV) if beta != 0 else torch.full(C.shape, float("nan"), device=DEV)
    lib.gemm(Ad, Bd, Cd, trans_a=ta, trans_b=tb, alpha=alpha, beta=beta, **opts)
    torch.cuda.synchronize()
    return Cd.cpu().numpy()


def check(oracle_mod, M, N, K, ta, tb, what, alpha=2.0, beta=-0.5, **opts):
    say(f"{what} M={M} N={N} K={K} ta={ta} tb={tb} alpha={alpha} beta={beta} opts={opts}")
    A, B, C = stored(M, N, K, ta, tb, "uniform", 500 + M + 3 * N + 7 * K)
    got = run_gemm(A, B, C, ta, tb, alpha, beta, **opts)
    ref, D = oracle_mod.gemm(A.numpy(), B.numpy(), C.numpy(), trans_a=ta, trans_b=tb, alpha=alpha, beta=beta,
                             with_denominator=True)
    assert_within_bound(got, ref, D, what=what)
    Ai, Bi, Ci = stored(M, N, K, ta, tb, "integer", 600 + M + 3 * N + 7 * K)
    goti = run_gemm(Ai, Bi, Ci, ta, tb, alpha, beta, **opts)
    refi = oracle_mod.gemm(Ai.numpy(), Bi.numpy(), Ci.numpy(), trans_a=ta, trans_b=tb, alpha=alpha, beta=beta)
    assert_bit_exact(goti, oracle_mod.round_to_f32(refi), what=what + " int")


SHAPES = [(300, 200, 20), (513, 385, 272), (1, 1, 1), (64, 8, 1000), (260, 300, 129)]
PLANS = [
    {},
    {"path": "mfma", "tile": 0, "decomposition": "tiles", "split_k": 1},
    {"path": "mfma", "tile": 0, "decomposition": "stream_k"},
    {"path": "mfma", "tile": 1, "decomposition": "tiles", "split_k": 1},
    {"path": "mfma", "tile": 1, "decomposition": "tiles", "split_k": 3},
    {"path": "mfma", "tile": 2, "decomposition": "tiles", "split_k": 1},
    {"path": "mfma", "tile": 2, "decomposition": "tiles", "split_k": 2},
    {"path": "mfma", "tile": 2, "decomposition": "stream_k"},
    {"path": "mfma", "tile": 3, "decomposition": "tiles", "split_k": 1},
    {"path": "mfma", "tile": 3, "decomposition": "stream_k"},
    {"path": "naive"},
]


@pytest.mark.parametrize("plan", PLANS, ids=lambda p: "-".join(f"{k}{v}" for k, v in p.items()) or "auto")
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=lambda v: str(int(v)))
def test_layouts_and_scalars(oracle_mod, ta, tb, shape, plan):
    check(oracle_mod, *shape, ta, tb, "gemm", **plan)


@pytest.mark.parametrize("tile", [0, 2])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=lambda v: str(int(v)))
def test_plain_product_matches_sgemm_bits(ta, tb, tile):
    """alpha = 1, beta = 0 on the same values: the NN call through sgemm_gemm
    returns the bits of sgemm; the transposed layouts agree with it within
    rounding (same tile, different fragment reads, same k order)."""
    M, N, K = 700, 520, 333
    say(f"gemm vs sgemm ta={ta} tb={tb} tile={tile}")
    A, B, _ = stored(M, N, K, False, False, "uniform", 71)
    Ad, Bd = A.to(DEV), B.to(DEV)
    C1 = lib.sgemm_ex(Ad, Bd, path="mfma", tile=tile, decomposition="tiles", split_k=1)
    As = A.t().contiguous().to(DEV) if ta else Ad
    Bs = B.t().contiguous().to(DEV) if tb else Bd
    C2 = lib.gemm(As, Bs, trans_a=ta, trans_b=tb, path="mfma", tile=tile, decomposition="tiles", split_k=1)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


@pytest.mark.parametrize("path,tile", [("valu", 0), ("skinny", -1), ("mfma", 0), ("mfma", 1), ("mfma", 2), ("mfma", 3)])
def test_scalars_on_every_path(oracle_mod, path, tile):
    M = 12 if path == "skinny" else 300
    for split in (1, 3):
        check(oracle_mod, M, 264, 200, False, False, f"{path}/{tile}/split{split}", path=path, tile=tile,
              split_k=split, alpha=-1.5, beta=0.25)
    if path == "skinny":       # alpha and beta applied by the stream-K fix-up and by whole strips
        check(oracle_mod, M, 264, 200, False, False, "skinny/stream_k", path=path, decomposition="stream_k",
              alpha=-1.5, beta=0.25)
        check(oracle_mod, 24, 700, 130, False, False, "skinny/stream_k/32", path=path, decomposition="stream_k",
              alpha=2.0, beta=-0.5)


def test_beta_zero_ignores_c_and_alpha_zero_ignores_ab(oracle_mod):
    say("scalar conventions")
    M, N, K = 300, 260, 100
    A, B, C = stored(M, N, K, False, True, "uniform", 81)
    Ad, Bd = A.to(DEV), B.to(DEV)
    Cd = torch.full((M, N), float("nan"), device=DEV)
    lib.gemm(Ad, Bd, Cd, trans_b=True, alpha=3.0, beta=0.0)
    torch.cuda.synchronize()
    ref, D = oracle_mod.gemm(A.numpy(), B.numpy(), trans_b=True, alpha=3.0, with_denominator=True)
    assert_within_bound(Cd.cpu().numpy(), ref, D, what="beta=0 with NaN C")
    nan_a = torch.full_like(Ad, float("nan"))
    nan_b = torch.full_like(Bd, float("nan"))
    Cd = C.to(DEV)
    lib.gemm(nan_a, nan_b, Cd, trans_b=True, alpha=0.0, beta=-2.0)
    torch.cuda.synchronize()
    assert np.array_equal(Cd.cpu().numpy(), (-2.0 * C).numpy())
    Cd = C.to(DEV)
    lib.gemm(nan_a, nan_b, Cd, trans_b=True, alpha=0.0, beta=0.0)
    torch.cuda.synchronize()
    c = Cd.cpu().numpy()
    assert np.all(c == 0) and not np.any(np.signbit(c))


@pytest.mark.parametrize("case", [
    (301, 260, 100, True, False),    # A stored K x M with M odd: A packed
    (300, 262, 100, False, False),   # N not a multiple of 4: B packed
    (300, 260, 101, False, True),    # K odd with B stored N x K: K padded, both packed
    (300, 260, 101, True, False),    # K odd, both operands k-major: no padding needed
    (301, 261, 99, True, True),
], ids=lambda c: "x".join(map(str, c[:3])) + f"_t{int(c[3])}{int(c[4])}")
@pytest.mark.parametrize("tile", [0, 2])
def test_packed_transposed_operands(oracle_mod, case, tile):
    M, N, K, ta, tb = case
    check(oracle_mod, M, N, K, ta, tb, f"packed tile {tile}", path="mfma", tile=tile, pack="always", split_k=1,
          decomposition="tiles")


def test_views_pick_the_layout():
    """A column-major view (W.t()) is passed as the stored matrix with op T:
    gemm(X, W.t()) is the same call as gemm(X, W, trans_b=True)."""
    say("views")
    X = workloads.draw(300, 200, "uniform", 91).to(DEV)
    W = workloads.draw(260, 200, "uniform", 92).to(DEV)
    C1 = lib.gemm(X, W.t())
    C2 = lib.gemm(X, W, trans_b=True)
    C3 = lib.gemm(W, X, trans_a=False, trans_b=True).t()      # (X W^T)^T = W X^T
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    ref = (X.double() @ W.double().t()).float()
    assert torch.allclose(C1, ref, rtol=0, atol=1e-4)
    assert torch.allclose(C3, ref, rtol=0, atol=1e-4)
    with pytest.raises(ValueError):
        lib.gemm(X, W)            # inner dimensions differ


def test_linear_layer_full_size(oracle_mod):
    """nn.Linear at the 8192 x 11008 x 4096 workload: X (M x K) . W^T with W
    stored N x K, as the default plan runs it; every element against the
    oracle's X . (W^T) (the same sums, W^T stored K x N row-major), and
    (X W^T) v = X (W^T v) on a probe vector."""
    w = workloads.CONFIGS["linear_8192x4096x11008"]
    say("linear NT full size")
    X = w.a()                                   # M x K
    Wt = w.b()                                  # K x N: W^T; store W = (W^T)^T row-major
    W = Wt.t().contiguous()                     # N x K
    plan = lib.gemm_plan_query("N", "T", w.M, w.N, w.K)
    assert plan["path_name"] == "mfma" and plan["vector"] == 1 and plan["packed"] == 0
    Cd = lib.gemm(X.to(DEV), W.to(DEV), trans_b=True)
    torch.cuda.synchronize()
    C = Cd.cpu().numpy()
    del Cd
    Xn, Wtn = X.numpy(), Wt.numpy()
    c_ref, d_ref = oracle_mod.sgemm(Xn, Wtn, with_denominator=True)
    e = assert_within_bound(C, c_ref, d_ref, what="linear N/T, every element")
    say(f"  max normalized error {e:.3e}")
    del c_ref, d_ref
    v = np.random.default_rng(6).uniform(-1, 1, size=w.N)
    lhs = np.empty(w.M)
    for r0 in range(0, w.M, 512):
        lhs[r0:r0 + 512] = C[r0:r0 + 512].astype(np.float64) @ v
    rhs = oracle_mod.gemv(Xn, oracle_mod.gemv(Wtn, v))
    scale = oracle_mod.gemv(Xn, oracle_mod.gemv(Wtn, np.abs(v), absolute=True), absolute=True)
    assert np.all(np.abs(lhs - rhs) <= 1e-5 * scale + 1e-12)


# --- the skinny path (M <= 32) in every operand layout ------------------------------------

SKINNY_LAYOUT_SHAPES = [
    (1, 1, 1),
    (5, 300, 1000),       # ragged N and K
    (16, 1000, 4100),     # K past a 64-deep step
    (17, 257, 129),       # two row blocks, N one past a strip
    (32, 65, 333),
    (9, 11008, 512),      # many strips
]
SKINNY_PLANS = [
    {"path": "skinny"},
    {"path": "skinny", "decomposition": "tiles", "split_k": 1},
    {"path": "skinny", "decomposition": "tiles", "split_k": 3},
    {"path": "skinny", "decomposition": "stream_k"},
    {"path": "skinny", "decomposition": "stream_k", "vector": 1},
]


@pytest.mark.parametrize("plan", SKINNY_PLANS, ids=lambda p: "-".join(f"{k}{v}" for k, v in p.items()))
@pytest.mark.parametrize("shape", SKINNY_LAYOUT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=lambda v: str(int(v)))
def test_skinny_layouts(oracle_mod, ta, tb, shape, plan):
    """The skinny kernel reads A stored K x M as single floats and B stored
    N x K as 16-byte runs along k (four k of one column per lane), in every
    decomposition, with alpha and beta."""
    M, N, K = shape
    q = lib.gemm_plan_query("T" if ta else "N", "T" if tb else "N", M, N, K, alpha=2.0, beta=-0.5, **plan)
    assert q["path_name"] == "skinny"
    check(oracle_mod, M, N, K, ta, tb, "skinny", **plan)


@pytest.mark.parametrize("case", [
    (513, 385, 272, {}),
    (80, 130, 70, {}),                                                  # 16 rows, K tail
    (96, 100, 300, {}),                                                 # 32 rows (two row blocks)
    (577, 301, 205, {"pack": "always"}),                               # packed operands
    (4097, 257, 1000, {"path": "mfma", "tile": 0}),
    (1040, 600, 900, {"path": "mfma", "tile": 2, "decomposition": "stream_k"}),
], ids=lambda c: "x".join(map(str, c[:3])))
@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)], ids=lambda v: str(int(v)))
def test_row_tail_transposed(oracle_mod, ta, tb, case):
    """The row tail with operands stored transposed: the skinny kernel takes
    rows M - r .. M - 1 of op(A) (columns of A stored K x M) after the main
    kernel."""
    M, N, K, opts = case
    q = lib.gemm_plan_query("T" if ta else "N", "T" if tb else "N", M, N, K, alpha=2.0, beta=-0.5,
                            row_tail="always", **opts)
    assert q["tail_rows"] == M % 64
    check(oracle_mod, M, N, K, ta, tb, "row tail", row_tail="always", **opts)


@pytest.mark.parametrize("kind", ["normal", "integer"])
def test_decode_linear_full_size(oracle_mod, kind):
    """The skinny workload in nn.Linear's layout: X (16 x 4096) . W^T with W
    stored 11008 x 4096, as the default plan (the skinny path) runs it; every
    element against the oracle."""
    say(f"decode linear N/T full size {kind}")
    M, N, K = 16, 11008, 4096
    X = workloads.draw(M, K, kind, 4242)
    W = workloads.draw(N, K, kind, 4243, std=(1.0 / 64 if kind == "normal" else 1.0))
    plan = lib.gemm_plan_query("N", "T", M, N, K)
    assert plan["path_name"] == "skinny" and plan["vector"] == 1
    Cd = lib.gemm(X.to(DEV), W.to(DEV), trans_b=True)
    torch.cuda.synchronize()
    C = Cd.cpu().numpy()
    ref, D = oracle_mod.gemm(X.numpy(), W.numpy(), trans_b=True, with_denominator=True)
    if kind == "integer":
        assert_bit_exact(C, oracle_mod.round_to_f32(ref), what="decode N/T integer, every element")
    else:
        assert_within_bound(C, ref, D, what="decode N/T, every element")


def _long_stride_dev(x, ld):
    """Device view of the CPU (rows, cols) tensor x with row stride ld; only
    the rows' own elements are written (the gap between them is never read)."""
    rows, cols = x.shape
    buf = torch.empty((rows - 1) * ld + cols, device=DEV)
    v = buf.as_strided((rows, cols), (ld, 1))
    v.copy_(x.to(DEV))
    return v


# Leading dimensions too long for the matrix-core loads' 32-bit lane offsets
# at some or every tile: (op A, op B, M, N, K, lda, ldb, forced plan, path
# taken).  The operands take several GB of device memory.
LONG_STRIDES = [
    (False, False, 300, 64, 48, 5_000_000, None, {}, "mfma"),                      # 128/64-row tiles as stored
    (False, False, 300, 64, 48, 5_000_000, None, {"path": "mfma", "tile": 0}, "mfma"),   # packed copy of A
    (False, False, 64, 64, 16, None, 72_000_000, {}, "mfma"),                      # k-major B, packed
    (False, False, 33, 4, 17_100_000, None, None, {}, "valu"),                      # K too long for any tile
    (False, True, 33, 4, 17_100_000, None, None, {}, "naive"),
]


@pytest.mark.parametrize("case", LONG_STRIDES, ids=lambda c: f"{'NT'[c[0]]}{'NT'[c[1]]}-{c[2]}x{c[3]}x{c[4]}-"
                         f"lda{c[5]}-ldb{c[6]}-{c[8]}-{'forced' if c[7] else 'auto'}")
def test_long_leading_dimensions(oracle_mod, case):
    """Products whose leading dimensions (or K) exceed what the matrix-core
    loads can address with 32-bit lane offsets give the oracle's result
    through a smaller tile, packed copies, or the 64-bit-addressed kernels."""
    ta, tb, M, N, K, lda, ldb, opts, path = case
    say(f"long strides ta={ta} tb={tb} M={M} N={N} K={K} lda={lda} ldb={ldb} opts={opts}")
    A, B, _ = stored(M, N, K, ta, tb, "uniform", 900 + M + N)
    Ad = _long_stride_dev(A, lda) if lda else A.to(DEV)
    Bd = _long_stride_dev(B, ldb) if ldb else B.to(DEV)
    p = lib.gemm_plan_query("T" if ta else "N", "T" if tb else "N", M, N, K, lda=Ad.stride(0), ldb=Bd.stride(0),
                            **opts)
    assert p["path_name"] == path, p
    C = torch.full((M, N), float("nan"), device=DEV)
    lib.gemm(Ad, Bd, C, trans_a=ta, trans_b=tb, **opts)
    torch.cuda.synchronize()
    del Ad, Bd
    torch.cuda.empty_cache()
    ref, D = oracle_mod.gemm(A.numpy(), B.numpy(), trans_a=ta, trans_b=tb, with_denominator=True)
    assert_within_bound(C.cpu().numpy(), ref, D, what=f"long strides {case}")
