"""GPU parity: the HIP kernels, called through the C interface, against the
host oracle on the same seeded inputs.

Bar (tests/checks.py): |C - C_ref| <= 1e-5 * sum_k |A_ik||B_kj| elementwise
for floating-point inputs; bit-exact on small-integer inputs, where every
partial sum is exact in FP32 whatever the order.
"""
import numpy as np
import pytest
import torch

import dense_fp32_matrix_amd as lib
import workloads
from checks import assert_bit_exact, assert_within_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)


def inputs(M, N, K, kind, seed, lda=None, ldb=None):
    A = workloads.with_ld(workloads.draw(M, K, kind, seed), lda or K)
    B = workloads.with_ld(workloads.draw(K, N, kind, seed + 1), ldb or N)
    return A, B


def to_dev(x):
    """Device copy keeping the row stride (padding included)."""
    if x.dim() == 2 and x.shape[0] > 0 and x.stride(0) != x.shape[1]:
        base = torch.empty((x.shape[0], x.stride(0)), dtype=torch.float32)
        base.fill_(float("nan"))
        base[:, :x.shape[1]] = x
        return base.to(DEV)[:, :x.shape[1]]
    return x.contiguous().to(DEV)


def run(A, B, ldc=None, **opts):
    Ad, Bd = to_dev(A), to_dev(B)
    M, N = A.shape[0], B.shape[1]
    if ldc is None:
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    else:
        C = torch.full((M, ldc), float("nan"), dtype=torch.float32, device=DEV)[:, :N]
    if opts:
        lib.sgemm_ex(Ad, Bd, C, **opts)
    else:
        lib.sgemm(Ad, Bd, C)
    torch.cuda.synchronize()
    return C


def check_case(oracle_mod, M, N, K, what, lda=None, ldb=None, **opts):
    say(f"{what} M={M} N={N} K={K} opts={opts}")
    # floating-point inputs: normalized bound
    A, B = inputs(M, N, K, "uniform", 100 + M + 7 * N + 13 * K, lda, ldb)
    C = run(A, B, **opts).cpu().numpy()
    Cref, D = oracle_mod.sgemm(A.numpy(), B.numpy(), with_denominator=True)
    assert_within_bound(C, Cref, D, what=what)
    # integer inputs: bit-exact
    Ai, Bi = inputs(M, N, K, "integer", 200 + M + 7 * N + 13 * K, lda, ldb)
    Ci = run(Ai, Bi, **opts).cpu().numpy()
    assert_bit_exact(Ci, oracle_mod.round_to_f32(oracle_mod.sgemm(Ai.numpy(), Bi.numpy())), what=what + " int")


# --- every path and tile on shapes that span several tiles with ragged tails ---------

SMALL_SHAPES = [
    (256, 256, 256),      # the 256^3 workload
    (300, 200, 20),       # the edge-handling example of the pages
    (1, 1, 1),
    (1, 65, 3),
    (33, 47, 65),
    (513, 385, 272),
    (130, 260, 100),
]


def _mfma_tiles():
    return list(range(lib.sgemm_tile_info("mfma", 0)["count"]))


def _narrow(tile):
    """Whether a matrix-core tile is built with 4-byte load lanes."""
    try:
        lib.sgemm_plan_query(64, 64, 64, path="mfma", tile=tile, vector=1)
        return True
    except lib.SgemmError:
        return False


def _mfma_variants():
    """(tile, vector) for every built instantiation: 16-byte lanes for all
    tiles, 4-byte lanes (vector=1) for the narrow ones."""
    return [(t, v) for t in _mfma_tiles() for v in (0, 1) if v == 0 or _narrow(t)]


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_naive(oracle_mod, shape):
    check_case(oracle_mod, *shape, "naive", path="naive")


@pytest.mark.parametrize("tile,vector", _mfma_variants())
@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_mfma_tiles(oracle_mod, shape, tile, vector):
    check_case(oracle_mod, *shape, f"mfma/{tile}/v{vector}", path="mfma", tile=tile, vector=vector, split_k=1,
               decomposition="tiles")


@pytest.mark.parametrize("tile", [0])
@pytest.mark.parametrize("vector", [0, 1])
@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_valu_tiles(oracle_mod, shape, tile, vector):
    check_case(oracle_mod, *shape, f"valu/{tile}/v{vector}", path="valu", tile=tile, vector=vector, split_k=1)


@pytest.mark.parametrize("vector", [0, 1])
@pytest.mark.parametrize("shape", [(1, 1, 1), (16, 64, 64), (5, 300, 1000), (16, 1000, 4100), (9, 11008, 512),
                                   (16, 7, 3), (17, 300, 1000), (32, 1000, 4100), (24, 65, 129), (32, 7, 3)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("split_k", [1, 3])
def test_skinny(oracle_mod, shape, vector, split_k):
    check_case(oracle_mod, *shape, f"skinny/v{vector}/s{split_k}", path="skinny", vector=vector, split_k=split_k)


@pytest.mark.parametrize("vector", [0, 1])
@pytest.mark.parametrize("shape", [
    (16, 3000, 1000),      # 47 strips x 16 K-steps over 256 workgroups: ranges straddle strips
    (5, 700, 333),         # one K-step per workgroup: every strip summed from six slots, K tail
    (32, 1000, 4100),      # two row blocks (tile 2)
    (16, 12800, 128),      # whole strips only: no partial strip, no fix-up
    (1, 1000, 200),        # a single row, K not a multiple of the step
], ids=lambda s: "x".join(map(str, s)))
def test_skinny_stream_k(oracle_mod, shape, vector):
    """The skinny kernel's stream-K decomposition (equal ranges of (strip,
    K-step) units, partial strips summed by the fix-up kernel)."""
    M, N, K = shape
    plan = lib.sgemm_plan_query(M, N, K, path="skinny", decomposition="stream_k", vector=vector)
    assert plan["decomposition_name"] == "stream_k" and plan["workgroups"] <= 512   # at most the workgroups the chip holds at once
    check_case(oracle_mod, M, N, K, f"skinny stream-K v{vector}", path="skinny", decomposition="stream_k",
               vector=vector)


@pytest.mark.parametrize("tile", list(range(lib.sgemm_tile_info("skinny", 0)["count"])))
def test_skinny_tiles(oracle_mod, tile):
    """Every skinny tile on the rows it holds (16, or 32 with two row blocks)."""
    M = lib.sgemm_tile_info("skinny", tile)["bm"]
    check_case(oracle_mod, M, 516, 2100, f"skinny tile {tile}", path="skinny", tile=tile, split_k=2)


SKINNY_EDGE_SHAPES = [(1, 1000, 200), (16, 64, 64), (5, 300, 1000), (16, 1000, 4100), (9, 11008, 512),
                      (16, 3000, 1000), (17, 300, 1000), (32, 1000, 4100), (24, 68, 132), (16, 12800, 128),
                      (32, 8, 4), (3, 4, 8)]


@pytest.mark.parametrize("decomposition,split", [("stream_k", 0), ("tiles", 1), ("tiles", 3)])
@pytest.mark.parametrize("shape", SKINNY_EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_skinny_edges(oracle_mod, shape, decomposition, split):
    """The skinny kernel in both decompositions on ragged shapes: stream-K
    ranges shorter than a strip and crossing strip boundaries, K tails inside
    a 64-deep unit, A rows past M and strips past N reading zeros."""
    M, N, K = shape
    opts = {"path": "skinny", "decomposition": decomposition}
    if split:
        opts["split_k"] = split
    check_case(oracle_mod, M, N, K, f"skinny {opts}", **opts)


@pytest.mark.parametrize("path,tile", [("mfma", 0), ("mfma", 1), ("mfma", 2), ("mfma", 3), ("valu", 0)])
@pytest.mark.parametrize("split_k", [2, 5, 16])
def test_split_k(oracle_mod, path, tile, split_k):
    check_case(oracle_mod, 200, 136, 2000, f"{path}/{tile}/split{split_k}", path=path, tile=tile,
               split_k=split_k)


STREAMK_SHAPES = [
    (300, 200, 20),        # fewer tiles than workgroups, one K-step per tile
    (513, 385, 1000),      # ragged tiles, K not a multiple of BK
    (1000, 1000, 3000),    # 16 tiles of 256x256 over 256 workgroups
    (4352, 4352, 48),      # 289 tiles: one data-parallel wave is not possible, all stream-K
    (4608, 4608, 32),      # 324 tiles: stream-K with whole tiles per workgroup
]


@pytest.mark.parametrize("tile,vector", _mfma_variants())
@pytest.mark.parametrize("shape", STREAMK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_stream_k(oracle_mod, shape, tile, vector):
    check_case(oracle_mod, *shape, f"streamk/{tile}/v{vector}", path="mfma", tile=tile, vector=vector,
               decomposition="stream_k")


@pytest.mark.parametrize("tile", _mfma_tiles())
def test_stream_k_after_data_parallel_tiles(oracle_mod, tile):
    """Stream-K where whole waves of tiles run data-parallel first (dp_tiles
    > 0) and the remaining tiles' K-steps are shared out in ranges that cut
    tiles (partial slots summed by the fix-up): the 8192 x 11008 x 4096
    workload's default plan in miniature, checked element by element."""
    M = N = 5888 if lib.sgemm_tile_info("mfma", tile)["bm"] == 256 else 2944
    K = 160
    plan = lib.sgemm_plan_query(M, N, K, path="mfma", tile=tile, decomposition="stream_k")
    assert plan["dp_tiles"] > 0 and plan["sk_tiles"] > 0 and plan["launches"] == 2, plan
    check_case(oracle_mod, M, N, K, f"streamk dp+sk tile {tile}", path="mfma", tile=tile, decomposition="stream_k")


@pytest.mark.parametrize("shape", SMALL_SHAPES + [(64, 64, 8192), (20, 11008, 4096)],
                         ids=lambda s: "x".join(map(str, s)))
def test_default_plan(oracle_mod, shape):
    check_case(oracle_mod, *shape, "auto")


@pytest.mark.parametrize("opts", [{"path": "mfma", "tile": 0, "decomposition": "tiles"},
                                  {"path": "mfma", "tile": 0, "decomposition": "stream_k"},
                                  {"path": "mfma", "tile": 2, "decomposition": "stream_k"},
                                  {"path": "mfma", "tile": 3, "decomposition": "tiles", "split_k": 3}],
                         ids=["tile0", "tile0-streamk", "tile2-streamk", "tile3-split3"])
def test_tile_order(oracle_mod, opts):
    """The plain row-major tile order (kept for comparing against the
    XCD-aware one).  With one tile per workgroup every tile is computed the
    same way in either order: identical bits.  Stream-K cuts the K-steps of
    the tiles in order, so there the order decides which tiles are split
    where: both results are checked against the oracle instead."""
    M, N, K = 1300, 1100, 700
    say(f"tile order {opts}")
    A, B = inputs(M, N, K, "uniform", 21)
    C1 = run(A, B, **opts).cpu()
    C2 = run(A, B, tile_order="plain", **opts).cpu()
    if opts["decomposition"] != "stream_k":
        assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))
    else:
        check_case(oracle_mod, M, N, K, "plain order", tile_order="plain", **opts)


# --- layouts: leading dimensions with NaN padding, misaligned bases -------------------------

@pytest.mark.parametrize("path", ["naive", "valu", "mfma", "skinny"])
def test_padded_leading_dimensions(oracle_mod, path):
    M = 16 if path == "skinny" else 150
    N, K = 170, 90
    lda, ldb, ldc = K + 3, N + 5, N + 7
    say(f"padded ld path={path}")
    A, B = inputs(M, N, K, "integer", 7, lda, ldb)
    C = run(A, B, ldc=ldc, path=path)
    Cbuf = C.cpu()  # the (M, N) view
    full = torch.as_strided(C, (M, ldc), (ldc, 1)).cpu().numpy()
    assert np.all(np.isnan(full[:, N:])), "wrote into the ldc gap"
    ref = oracle_mod.round_to_f32(oracle_mod.sgemm(A.numpy(), B.numpy()))
    assert_bit_exact(Cbuf.numpy(), ref, what=f"{path} padded")


@pytest.mark.parametrize("tile", _mfma_tiles())
@pytest.mark.parametrize("gap", [4, 7], ids=["ldc16B", "ldcodd"])
def test_epilogue_keeps_ldc_gap(oracle_mod, tile, gap):
    """Each tile's epilogue (the 16-byte interleaved-column stores of the
    256 x 256 tiles included) writes exactly [0, M) x [0, N): the NaN gap of a
    padded ldc survives, with N ragged against the tile and against 4 columns."""
    M, N, K = 300, 270, 100
    ldc = N + gap
    say(f"ldc gap tile={tile} ldc={ldc}")
    A, B = inputs(M, N, K, "integer", 11)
    C = run(A, B, ldc=ldc, path="mfma", tile=tile, decomposition="tiles", split_k=1)
    full = torch.as_strided(C, (M, ldc), (ldc, 1)).cpu().numpy()
    assert np.all(np.isnan(full[:, N:])), "wrote into the ldc gap"
    ref = oracle_mod.round_to_f32(oracle_mod.sgemm(A.numpy(), B.numpy()))
    assert_bit_exact(full[:, :N], ref, what=f"tile {tile} ldc {ldc}")


@pytest.mark.parametrize("path,pack", [("valu", "never"), ("mfma", "never"), ("mfma", "always"),
                                       ("skinny", "never")])
def test_misaligned_base_pointers(oracle_mod, path, pack):
    """Views starting one float into their buffers: 4-byte aligned only."""
    M = 12 if path == "skinny" else 97
    N, K = 132, 76
    say(f"misaligned path={path} pack={pack}")
    A, B = inputs(M, N, K, "integer", 9)
    Abuf = torch.zeros((M * K + 1,), dtype=torch.float32, device=DEV)
    Bbuf = torch.zeros((K * N + 1,), dtype=torch.float32, device=DEV)
    Cbuf = torch.full((M * N + 2,), float("nan"), dtype=torch.float32, device=DEV)
    Ad = Abuf[1:].view(M, K)
    Bd = Bbuf[1:].view(K, N)
    Cd = Cbuf[1:M * N + 1].view(M, N)
    Ad.copy_(A.to(DEV))
    Bd.copy_(B.to(DEV))
    plan = lib.sgemm_plan_query(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N, Cd.data_ptr(), N, path=path,
                                pack=pack)
    if pack == "always":
        assert plan["vector"] == 1 and plan["packed"] == 3
    else:
        assert plan["vector"] == 0 and plan["packed"] == 0
    lib.sgemm_ex(Ad, Bd, Cd, path=path, pack=pack)
    torch.cuda.synchronize()
    c = Cbuf.cpu().numpy()
    assert np.isnan(c[0]) and np.isnan(c[-1]), "wrote outside C"
    ref = oracle_mod.round_to_f32(oracle_mod.sgemm(A.numpy(), B.numpy()))
    assert_bit_exact(c[1:M * N + 1].reshape(M, N), ref, what=f"{path} misaligned")


# --- packed operands: misaligned operands copied to aligned, zero-padded workspace -------------

PACK_CASES = [
    # (M, N, K, lda, ldb, packed bits expected)
    (300, 200, 21, None, None, 3),      # K not a multiple of 4: both operands padded along K
    (130, 261, 100, None, None, 2),     # N odd: B only
    (130, 260, 100, 101, None, 1),      # lda odd: A only
    (513, 385, 272, 273, 387, 3),       # both leading dimensions odd, NaN in the gaps
    (1, 1, 1, None, None, 3),
    (600, 517, 333, 335, None, 3),      # several 256 x 256 tiles, ragged in every dimension
    (70, 40, 4501, None, None, 3),      # A rows of 1126 16-byte groups (two packing pieces), B rows of 10
    (97, 4099, 33, 35, 4101, 3),        # B rows of 1025 groups (a one-group second piece), A rows of 9
]


@pytest.mark.parametrize("tile", _mfma_tiles())
@pytest.mark.parametrize("decomposition", ["tiles", "stream_k"])
@pytest.mark.parametrize("case", PACK_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"_lda{c[3]}_ldb{c[4]}")
def test_packed_operands(oracle_mod, case, decomposition, tile):
    """Packed copies on every tile in both decompositions (the ragged
    workload's default plan is packed operands on the 128 x 128 tile with
    stream-K)."""
    M, N, K, lda, ldb, bits = case
    plan = lib.sgemm_plan_query(M, N, K, lda=lda or K, ldb=ldb or N, path="mfma", tile=tile, pack="always",
                                decomposition=decomposition)
    assert plan["packed"] == bits and plan["vector"] == 1
    assert plan["k_padded"] == (K + 3) // 4 * 4
    check_case(oracle_mod, M, N, K, f"packed/{decomposition}/tile{tile}", lda=lda, ldb=ldb, path="mfma", tile=tile,
               pack="always", decomposition=decomposition)


# --- the row tail: the last 1-32 rows of M through the skinny kernel ------------------------

ROW_TAIL_CASES = [  # M, N, K, lda, ldb, forced main options
    (513, 385, 272, None, None, {}),                                   # one row, 64x64 tile
    (65, 64, 64, None, None, {}),                                      # one row past one tile
    (80, 130, 70, None, None, {}),                                     # 16 rows (skinny tile 0), K tail
    (96, 100, 300, None, None, {}),                                    # 32 rows (skinny tile 1)
    (113, 200, 3000, None, None, {}),                                  # 49 rows: no tail (beyond 32)
    (577, 301, 205, 205, 301, {}),                                     # packed operands, one row
    (4097, 257, 1000, None, None, {"path": "mfma", "tile": 0}),       # 256x256 main tile
    (1040, 600, 900, None, None, {"path": "mfma", "tile": 2, "decomposition": "stream_k"}),
    (1040, 600, 900, None, None, {"path": "mfma", "tile": 3, "split_k": 3}),
]


@pytest.mark.parametrize("case", ROW_TAIL_CASES, ids=lambda c: "x".join(map(str, c[:3])) + str(c[5]))
def test_row_tail(oracle_mod, case):
    """row_tail = always: the main kernel takes the rows up to the last
    multiple of 64, the skinny kernel the 1-32 rows after them (its own
    split-K or stream-K plan), on aligned and packed operands and with the
    main kernel's tile and decomposition forced."""
    M, N, K, lda, ldb, opts = case
    plan = lib.sgemm_plan_query(M, N, K, lda=lda or K, ldb=ldb or N, row_tail="always", **opts)
    r = M % 64
    assert plan["tail_rows"] == (r if 1 <= r <= 32 else 0), plan
    check_case(oracle_mod, M, N, K, f"row tail {opts}", lda=lda, ldb=ldb, row_tail="always", **opts)


def test_row_tail_with_alpha_beta(oracle_mod):
    """The tail applies alpha and beta to its rows as the main kernel does to the others."""
    M, N, K = 257, 300, 500
    say("row tail alpha/beta")
    A, B = inputs(M, N, K, "integer", 91)
    C0 = workloads.draw(M, N, "integer", 92)
    Cd = C0.to(DEV)
    lib.gemm(to_dev(A), to_dev(B), Cd, alpha=2.0, beta=-0.5, row_tail="always")
    torch.cuda.synchronize()
    assert lib.gemm_plan_query("N", "N", M, N, K, alpha=2.0, beta=-0.5, row_tail="always")["tail_rows"] == 1
    ref = oracle_mod.gemm(A.numpy(), B.numpy(), C0.numpy(), alpha=2.0, beta=-0.5)
    assert_bit_exact(Cd.cpu().numpy(), oracle_mod.round_to_f32(ref), what="row tail alpha/beta")


def test_packed_matches_unpacked_bits():
    """Packing copies values exactly and pads with zeros: the 16-byte kernel
    on packed copies returns the bits of the 16-byte kernel run on an
    aligned copy of the same operands made on the host."""
    M, N, K = 700, 301, 517
    say("packed vs aligned copy")
    A, B = inputs(M, N, K, "uniform", 77)
    Kp, Np = 520, 304
    Ap = torch.zeros((M, Kp)); Ap[:, :K] = A
    Bp = torch.zeros((Kp, Np)); Bp[:K, :N] = B
    C1 = run(A, B, path="mfma", tile=0, pack="always", decomposition="tiles")
    C2 = run(Ap, Bp[:, :N], path="mfma", tile=0, decomposition="tiles")
    assert torch.equal(C1.cpu(), C2.cpu())


# --- degenerate sizes ------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["auto", "naive", "valu", "mfma"])
def test_k_zero_writes_zeros(path):
    say(f"K=0 path={path}")
    A = torch.empty((5, 0), device=DEV)
    B = torch.empty((0, 7), device=DEV)
    C = torch.full((5, 7), float("nan"), device=DEV)
    lib.sgemm_ex(A, B, C, path=path)
    torch.cuda.synchronize()
    c = C.cpu().numpy()
    assert np.all(c == 0) and not np.any(np.signbit(c))


def test_empty_m_or_n_is_noop():
    say("M=0 / N=0")
    C = torch.full((0, 7), 1.0, device=DEV)
    lib.sgemm(torch.empty((0, 3), device=DEV), torch.ones((3, 7), device=DEV), C)
    C2 = torch.full((4, 0), 1.0, device=DEV)
    lib.sgemm(torch.ones((4, 3), device=DEV), torch.empty((3, 0), device=DEV), C2)
    torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["naive", "valu", "mfma", "skinny"])
def test_k_one_single_rounding(oracle_mod, path):
    """K = 1: each output is one rounded product, equal to the binary32 product."""
    M = 16 if path == "skinny" else 77
    say(f"K=1 path={path}")
    A, B = inputs(M, 91, 1, "uniform", 11)
    C = run(A, B, path=path).cpu().numpy()
    ref = oracle_mod.round_to_f32(oracle_mod.sgemm(A.numpy(), B.numpy()))
    assert_bit_exact(C, ref, what=f"{path} K=1")
    assert_bit_exact(C, A.numpy() * B.numpy(), what=f"{path} K=1 vs fp32 product")


def test_zero_row_and_column_exact(oracle_mod):
    """Where D = 0 (a zero row of A or zero column of B) C must be exactly 0."""
    say("zero row/column")
    A, B = inputs(130, 140, 150, "uniform", 12)
    A[5] = 0
    B[:, 17] = 0
    C = run(A, B).cpu().numpy()
    assert np.all(C[5] == 0) and np.all(C[:, 17] == 0)


@pytest.mark.parametrize("opts", [{}, {"path": "mfma", "tile": 2, "split_k": 4}, {"path": "skinny"},
                                  {"path": "mfma", "tile": 3, "decomposition": "stream_k"}],
                         ids=["auto", "split4", "skinny", "streamk"])
def test_run_to_run_determinism(opts):
    say(f"determinism {opts}")
    M = 16 if opts.get("path") == "skinny" else 300
    A, B = inputs(M, 500, 3000, "uniform", 13)
    C1 = run(A, B, **opts).cpu()
    C2 = run(A, B, **opts).cpu()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))


def test_caller_workspace_and_stream(oracle_mod):
    say("caller workspace + side stream")
    M, N, K = 200, 136, 2000
    A, B = inputs(M, N, K, "integer", 14)
    need = lib.sgemm_plan_query(M, N, K, path="mfma", tile=2, split_k=4)["workspace_bytes"]
    ws = torch.empty(need // 4 + 64, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    Ad, Bd = to_dev(A), to_dev(B)
    C = torch.empty((M, N), device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        lib.sgemm_ex(Ad, Bd, C, stream=s, path="mfma", tile=2, split_k=4, workspace=ws)
    s.synchronize()
    ref = oracle_mod.round_to_f32(oracle_mod.sgemm(A.numpy(), B.numpy()))
    assert_bit_exact(C.cpu().numpy(), ref, what="caller workspace")
    small = torch.empty(16, dtype=torch.float32, device=DEV)
    with pytest.raises(lib.SgemmError):
        lib.sgemm_ex(Ad, Bd, C, path="mfma", tile=2, split_k=4, workspace=small)


def test_library_workspace_reuse(oracle_mod):
    """Calls without a caller workspace share one library-held buffer per
    stream: growing requests, shrinking ones and two streams in turn, with
    nothing synchronised between the calls, each checked bit-exact."""
    cases = [((200, 136, 2000), {"path": "mfma", "tile": 2, "split_k": 4}),
             ((600, 517, 700), {"path": "mfma", "tile": 1, "decomposition": "stream_k"}),
             ((1000, 900, 3000), {"path": "mfma", "tile": 2, "split_k": 6, "decomposition": "tiles"}),
             ((16, 700, 5000), {"path": "skinny", "split_k": 3}),
             ((300, 260, 900), {"path": "mfma", "tile": 3, "decomposition": "stream_k"})]
    side = torch.cuda.Stream()
    jobs = []
    for i, ((M, N, K), opts) in enumerate(cases * 2):
        A, B = inputs(M, N, K, "integer", 40 + i)
        jobs.append((A, B, to_dev(A), to_dev(B), torch.full((M, N), float("nan"), device=DEV), opts, i % 2))
    torch.cuda.synchronize()
    for A, B, Ad, Bd, C, opts, on_side in jobs:
        say(f"workspace reuse {tuple(C.shape)} {opts} side={on_side}")
        if on_side:
            with torch.cuda.stream(side):
                lib.sgemm_ex(Ad, Bd, C, stream=side, **opts)
        else:
            lib.sgemm_ex(Ad, Bd, C, **opts)
    torch.cuda.synchronize()
    for A, B, Ad, Bd, C, opts, on_side in jobs:
        ref = oracle_mod.round_to_f32(oracle_mod.sgemm(A.numpy(), B.numpy()))
        assert_bit_exact(C.cpu().numpy(), ref, what=f"workspace reuse {opts}")


def test_workspace_on_many_streams(oracle_mod):
    """More streams than the library keeps buffers for (8 per device): the
    calls on the further streams allocate their own; all run concurrently,
    unsynchronised, and every result is bit-exact."""
    M, N, K = 260, 300, 1500
    opts = {"path": "mfma", "tile": 3, "split_k": 4, "decomposition": "tiles"}
    streams = [torch.cuda.Stream() for _ in range(11)]
    jobs = []
    for i, st in enumerate(streams):
        A, B = inputs(M, N, K, "integer", 80 + i)
        jobs.append((A, B, to_dev(A), to_dev(B), torch.full((M, N), float("nan"), device=DEV), st))
    torch.cuda.synchronize()
    for rep in range(2):
        say(f"many streams, round {rep}")
        for A, B, Ad, Bd, C, st in jobs:
            with torch.cuda.stream(st):
                lib.sgemm_ex(Ad, Bd, C, stream=st, **opts)
        torch.cuda.synchronize()
        for A, B, Ad, Bd, C, st in jobs:
            ref = oracle_mod.round_to_f32(oracle_mod.sgemm(A.numpy(), B.numpy()))
            assert_bit_exact(C.cpu().numpy(), ref, what=f"many streams round {rep}")
            C.fill_(float("nan"))
        torch.cuda.synchronize()


def test_large_workspace_allocated_per_call(oracle_mod):
    """A split-K workspace above the library's cached limit (1 GiB of slices
    here) is allocated and freed with the call; every element checked,
    twice in a row."""
    M, N, K = 4096, 4096, 8192
    opts = {"path": "mfma", "tile": 1, "split_k": 16, "decomposition": "tiles"}
    assert lib.sgemm_plan_query(M, N, K, **opts)["workspace_bytes"] > (512 << 20)
    A, B = inputs(M, N, K, "integer", 70)
    Ad, Bd = to_dev(A), to_dev(B)
    ref = oracle_mod.round_to_f32(oracle_mod.sgemm(A.numpy(), B.numpy()))
    for r in range(2):
        say(f"large workspace call {r}")
        C = torch.full((M, N), float("nan"), device=DEV)
        lib.sgemm_ex(Ad, Bd, C, **opts)
        torch.cuda.synchronize()
        assert_bit_exact(C.cpu().numpy(), ref, what=f"large workspace call {r}")
        del C


@pytest.mark.parametrize("opts", [{"path": "mfma", "tile": 2, "split_k": 4, "decomposition": "tiles"},
                                  {"path": "mfma", "tile": 3, "decomposition": "stream_k"}, {},
                                  {"path": "skinny", "decomposition": "stream_k"}],
                         ids=["split4", "streamk", "auto", "skinny-streamk"])
def test_graph_capture_replays(oracle_mod, opts):
    """A call captured into a graph (its workspace then belongs to the graph,
    not to the library's per-stream buffer) replays correctly: new inputs are
    copied in eagerly between replays, and every replay is checked."""
    say(f"graph capture {opts}")
    M, N, K = (24, 700, 1100) if opts.get("path") == "skinny" else (520, 390, 1100)
    Ad = torch.empty((M, K), device=DEV)
    Bd = torch.empty((K, N), device=DEV)
    C = torch.empty((M, N), device=DEV)
    A0, B0 = inputs(M, N, K, "integer", 60)
    Ad.copy_(A0)
    Bd.copy_(B0)
    lib.sgemm_ex(Ad, Bd, C, **opts)           # eager call first (plans and library workspace in place)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.sgemm_ex(Ad, Bd, C, **opts)
    torch.cuda.synchronize()
    for r in range(3):
        A, B = inputs(M, N, K, "integer", 61 + r)
        Ad.copy_(A)
        Bd.copy_(B)
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle_mod.round_to_f32(oracle_mod.sgemm(A.numpy(), B.numpy()))
        assert_bit_exact(C.cpu().numpy(), ref, what=f"graph replay {r} {opts}")
        lib.sgemm_ex(Ad, Bd, C, **opts)       # eager work between replays
        torch.cuda.synchronize()
        assert_bit_exact(C.cpu().numpy(), ref, what=f"eager after replay {r} {opts}")


# --- the benchmark workloads at full size, in the benchmark's launch configuration ---------

def _full_size_check(oracle_mod, w, kind, opts=None):
    """The whole output against the whole oracle product, element by element:
    within the normalized bound on floating-point inputs, bit-exact on
    integer ones.  (AB)x = A(Bx) on two probe vectors is checked as well."""
    say(f"full size {w.name} inputs={kind} opts={opts}")
    A = workloads.with_ld(workloads.draw(w.M, w.K, kind, w.seed_base + 0, w.a_std if kind != "integer" else 1.0),
                          w.lda)
    B = workloads.with_ld(workloads.draw(w.K, w.N, kind, w.seed_base + 1, w.b_std if kind != "integer" else 1.0),
                          w.ldb)
    Ad, Bd = to_dev(A), to_dev(B)
    C = torch.full((w.M, w.N), float("nan"), dtype=torch.float32, device=DEV)
    if opts:
        lib.sgemm_ex(Ad, Bd, C, **opts)
    else:
        lib.sgemm(Ad, Bd, C)             # the default plan, as the benchmark runs it
    torch.cuda.synchronize()
    del Ad, Bd
    Ch = C.cpu().numpy()
    del C
    An, Bn = A.numpy(), B.numpy()
    if kind == "integer":
        Cref = oracle_mod.sgemm(An, Bn)
        assert_bit_exact(Ch, oracle_mod.round_to_f32(Cref), what=f"{w.name} integer, every element")
    else:
        Cref, D = oracle_mod.sgemm(An, Bn, with_denominator=True)
        e = assert_within_bound(Ch, Cref, D, what=f"{w.name} {kind}, every element")
        say(f"  max normalized error {e:.3e}")
        del D
    del Cref
    # (AB)x = A(Bx) over the whole output, for two vectors x
    g = np.random.default_rng(w.seed_base + 9)
    for t in range(2):
        if kind == "integer":
            x = g.integers(-4, 5, size=w.N).astype(np.float64)
        else:
            x = g.uniform(-1, 1, size=w.N)
        cx = np.empty(w.M)
        for r0 in range(0, w.M, 512):
            cx[r0:r0 + 512] = Ch[r0:r0 + 512].astype(np.float64) @ x
        abx = oracle_mod.gemv(An, oracle_mod.gemv(Bn, x))
        if kind == "integer":
            assert np.array_equal(cx, abx), "(AB)x != A(Bx) on integer inputs"
        else:
            scale = oracle_mod.gemv(An, oracle_mod.gemv(Bn, np.abs(x), absolute=True), absolute=True)
            r = np.abs(cx - abx) / scale
            assert r.max() <= 1e-5 + 1e-12, f"(AB)x vs A(Bx): {r.max():.3e}"


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_full_size_workload(oracle_mod, name):
    w = workloads.CONFIGS[name]
    _full_size_check(oracle_mod, w, w.a_kind)


@pytest.mark.parametrize("kind", ["normal", "integer"])
def test_full_size_skinny_stream_k(oracle_mod, kind):
    """The skinny workload at full size through the skinny stream-K plan (a
    persistent grid of every resident workgroup, the shared strips summed in
    workgroup order), every element checked."""
    w = workloads.CONFIGS["linear_skinny_16x4096x11008"]
    _full_size_check(oracle_mod, w, kind, {"path": "skinny", "decomposition": "stream_k"})


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_full_size_workload_integer(oracle_mod, name):
    w = workloads.CONFIGS[name]
    _full_size_check(oracle_mod, w, "integer")


@pytest.mark.parametrize("n", [0, 4, 1 << 20, (1 << 20) + 4 * 1021, 3 * 1024 * 1024 + 8])
def test_read_probe(n):
    """The read-rate probe reads every element once: on small integers its
    per-workgroup sums are exact, and together they give the buffer's sum
    (chunks that end inside the unrolled loads, workgroups left without a
    chunk, and the empty buffer included)."""
    say(f"read probe n={n}")
    g = torch.Generator().manual_seed(n + 3)
    x = torch.randint(0, 3, (n,), generator=g, dtype=torch.int32).to(torch.float32)
    part = lib.read_probe(x.to(DEV))
    torch.cuda.synchronize()
    p = part.cpu().to(torch.float64)
    assert part.numel() == lib.READ_PROBE_PARTIALS
    assert torch.equal(p, p.round()) and int(p.sum().item()) == int(x.to(torch.int64).sum().item())


def test_fma_probe_values():
    """The FMA-rate probe computes what it claims: with no iterations each lane
    holds the sum of its chains' starting values (0 + 1 + ... + 15); with i
    iterations each of the 16 chains gained 8 i products x * y."""
    say("fma probe")
    out0 = lib.fma_probe(0, 2)
    out3 = lib.fma_probe(3, 2)
    torch.cuda.synchronize()
    assert torch.all(out0.cpu() == 120.0)
    lane = torch.arange(512) % 256
    wg = torch.arange(512) // 256
    x = (1.0 + 1e-7 * lane.double())
    y = (1.0 - 1e-7 * wg.double())
    expect = 120.0 + 16 * 8 * 3 * x * y
    assert torch.allclose(out3.cpu().double(), expect, rtol=1e-5, atol=0)
