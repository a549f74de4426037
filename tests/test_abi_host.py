"""Host-only checks of the C interface: the library loads, exports what the
header declares, rejects bad arguments before any HIP call, and plans
launches as the tile arithmetic says.  No compute runs here."""
import ctypes
import json
import os
import re
import subprocess

import pytest

import dense_fp32_matrix_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(sgemm[a-z_0-9]*)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"sgemm", "sgemm_ex", "sgemm_plan_query", "sgemm_workspace_size", "sgemm_tile_info",
            "sgemm_status_string", "sgemm_version", "sgemm_read_probe", "sgemm_fma_probe"} <= set(names)
    so = ctypes.CDLL(lib.library_path())
    for n in names:
        assert hasattr(so, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lib.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported


def test_header_is_valid_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "sgemm.h"\nint main(void){ sgemm_options o = {0}; (void)o; '
                   'return (int)sizeof(sgemm_plan) > 0 ? 0 : 1; }\n')
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                    f"-I{os.path.join(ROOT, 'include')}", "-I/opt/rocm/include", str(src)], check=True)


def test_status_strings_and_version():
    assert lib.sgemm_status_string(0) == "SGEMM_OK"
    assert lib.sgemm_status_string(1).startswith("SGEMM_ERR_INVALID_ARG")
    assert lib.sgemm_status_string(99) == "unknown sgemm_status"
    assert re.fullmatch(r"\d+\.\d+\.\d+", lib.sgemm_version())


# Arguments are rejected on the host: with fake, never-dereferenced addresses
# the calls below must return an error code without reaching the GPU.
A, B, C = 0x10000000, 0x20000000000, 0x30000000000


@pytest.mark.parametrize("args,status", [
    ((-1, 4, 4, A, 4, B, 4, C, 4), 1),            # negative M
    ((4, -1, 4, A, 4, B, 4, C, 4), 1),            # negative N
    ((4, 4, -1, A, 4, B, 4, C, 4), 1),            # negative K
    ((4, 4, 8, A, 7, B, 4, C, 4), 1),             # lda < K
    ((4, 8, 4, A, 4, B, 7, C, 8), 1),             # ldb < N
    ((4, 8, 4, A, 4, B, 8, C, 7), 1),             # ldc < N
    ((4, 4, 4, 0, 4, B, 4, C, 4), 1),             # A NULL with M, K > 0
    ((4, 4, 4, A, 4, 0, 4, C, 4), 1),             # B NULL with K, N > 0
    ((4, 4, 4, A, 4, B, 4, 0, 4), 1),             # C NULL with M, N > 0
    ((4, 4, 4, A + 2, 4, B, 4, C, 4), 1),         # A not 4-byte aligned
    ((4, 4, 4, A, 4, B, 4, A + 8, 4), 1),         # C overlaps A
    ((4, 4, 4, A, 4, B, 4, B + 60, 4), 1),        # C overlaps the end of B
    ((1 << 30, 4, 4, A, 4, B, 4, C, 4), 2),       # beyond the kernels' index range
])
def test_invalid_arguments_rejected_before_hip(args, status):
    assert lib.sgemm_raw(*args, stream=0) == status
    assert lib.sgemm_raw(*args, stream=0, opts=lib._options()) == status


@pytest.mark.parametrize("args,status", [
    ((2, 0, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4), 1),       # op_a not N or T
    ((0, -1, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4), 1),      # op_b not N or T
    ((1, 0, 8, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4), 1),       # A stored K x M needs lda >= M
    ((0, 1, 4, 4, 8, 1.0, A, 8, B, 4, 0.0, C, 4), 1),       # B stored N x K needs ldb >= K
    ((0, 1, 4, 4, 8, 1.0, A, 8, B, 8, 0.0, C + 2, 4), 1),   # C misaligned
    ((1, 1, 4, 4, 4, 1.0, 0, 4, B, 4, 0.0, C, 4), 1),       # A NULL while read
    ((0, 0, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, A + 8, 4), 1),   # C overlaps A
])
def test_gemm_invalid_arguments(args, status):
    assert lib.gemm_raw(*args, stream=0) == status


def test_gemm_plans():
    """Operand layouts and scalars in the plan: transposed operands run on the
    direct-to-LDS tiles; alpha == 0 or K == 0 is one scaling launch that
    reads neither A nor B (NULL allowed); the alignment rule follows each
    operand's contiguous dimension."""
    M, N, K = 8192, 11008, 4096
    p = lib.gemm_plan_query("N", "T", M, N, K)                   # nn.Linear: X . W^T
    assert p["path_name"] == "mfma" and (p["bm"], p["bn"]) == (256, 256) and p["vector"] == 1 and p["packed"] == 0
    for ops in [("T", "N"), ("T", "T"), ("N", "T")]:
        q = lib.gemm_plan_query(*ops, 4096, 4096, 4096)
        assert (q["bm"], q["bn"]) == (256, 256) and q["vector"] == 1
    # alpha == 0: C = beta * C only, A and B may be NULL
    q = lib.gemm_plan_query("N", "N", 64, 64, 64, alpha=0.0, A=0, B=0, beta=2.0)
    assert q["launches"] == 1 and q["workspace_bytes"] == 0
    # k-major operands (A stored K x M, B stored K x N) need no K padding for odd K
    q = lib.gemm_plan_query("T", "N", 512, 512, 511, path="mfma", tile=0, split_k=1, decomposition="tiles")
    assert q["vector"] == 1 and q["packed"] == 0 and q["k_padded"] == 511
    # odd K with a k-contiguous operand: pads K, packs both
    q = lib.gemm_plan_query("N", "T", 512, 512, 511, path="mfma", tile=0, split_k=1, decomposition="tiles",
                            pack="always")
    assert q["packed"] == 3 and q["k_padded"] == 512
    # the VALU path reads operands as stored only
    with pytest.raises(lib.SgemmError):
        lib.gemm_plan_query("N", "T", 16, 512, 512, path="valu")
    assert lib.gemm_plan_query("T", "T", 300, 200, 20, path="naive")["path_name"] == "naive"
    # M <= 32 in every layout: the skinny path; its 16-byte loads need B's rows
    # (k-contiguous when B is transposed) and, as stored, A's rows aligned
    for ops in [("N", "T"), ("T", "N"), ("T", "T")]:
        for m in (1, 16, 32):
            q = lib.gemm_plan_query(*ops, m, 11008, 4096)
            assert q["path_name"] == "skinny" and q["vector"] == 1, (ops, m, q)
    assert lib.gemm_plan_query("N", "T", 16, 11008, 4095)["vector"] == 0          # odd K: B's rows misaligned
    assert lib.gemm_plan_query("T", "N", 16, 11008, 4095, lda=17)["vector"] == 1  # A read as single floats
    assert lib.gemm_plan_query("N", "N", 16, 11008, 4095)["vector"] == 0          # A's rows misaligned
    assert lib.gemm_workspace_size("N", "T", M, N, K) == p["workspace_bytes"]


def test_bad_options_rejected():
    base = (64, 64, 64, A, 64, B, 64, C, 64)
    assert lib.sgemm_raw(*base, opts=lib._options(path=7)) == 1
    assert lib.sgemm_raw(*base, opts=lib._options(path="mfma", tile=99)) == 1
    assert lib.sgemm_raw(*base, opts=lib._options(split_k=-2)) == 1
    assert lib.sgemm_raw(*base, opts=lib._options(path="skinny")) == 1          # M > 32
    few = (20, 64, 64, A, 64, B, 64, C, 64)
    assert lib.sgemm_raw(*few, opts=lib._options(path="skinny", tile=0)) == 1   # tile 0 holds 16 rows
    # skinny stream-K: both tiles, and no split-K with it
    sk = (16, 64, 640)
    for tile in (0, 1):
        assert lib.sgemm_plan_query(*sk, path="skinny", tile=tile, decomposition="stream_k")["decomposition_name"] \
            == "stream_k"
    with pytest.raises(lib.SgemmError):
        lib.sgemm_plan_query(*sk, path="skinny", decomposition="stream_k", split_k=2)
    with pytest.raises(lib.SgemmError):
        lib.sgemm_plan_query(*sk, path="valu", decomposition="stream_k")
    assert lib.sgemm_raw(*base, opts=lib._options(path="naive", split_k=2)) == 1
    assert lib.sgemm_raw(*base, opts=lib._options(workspace=A + 16, workspace_bytes=1 << 20)) == 1
    assert lib.sgemm_raw(*base, opts=lib._options(pack=-1)) == 1
    assert lib.sgemm_raw(*base, opts=lib._options(tile_order=2)) == 1


def test_wide_tiles_have_no_narrow_lanes():
    """The 256 x 256 tiles are built for 16-byte lanes only: forcing them with
    4-byte lanes, or on unaligned operands with packing off, is an invalid
    argument; on unaligned operands with packing allowed they run on packed
    copies; the 128 x 128 and 64 x 64 tiles take 4-byte lanes."""
    for tile in (0, 1):
        with pytest.raises(lib.SgemmError):
            lib.sgemm_plan_query(512, 512, 512, path="mfma", tile=tile, vector=1)
        with pytest.raises(lib.SgemmError):
            lib.sgemm_plan_query(512, 509, 512, path="mfma", tile=tile, pack="never")
        p = lib.sgemm_plan_query(512, 509, 512, path="mfma", tile=tile)
        assert p["tile"] == tile and p["vector"] == 1 and p["packed"] == 2
    for tile in (2, 3):
        p = lib.sgemm_plan_query(512, 512, 512, path="mfma", tile=tile, vector=1)
        assert p["tile"] == tile and p["vector"] == 0 and p["packed"] == 0
    # unaligned operands with packing off: the planner picks a tile with 4-byte lanes
    p = lib.sgemm_plan_query(4097, 3001, 2049, lda=2049, ldb=3001, ldc=3001, pack="never")
    assert p["path_name"] == "mfma" and p["vector"] == 0 and p["tile"] in (2, 3)


def test_empty_problems_plan_no_launch():
    assert lib.sgemm_plan_query(0, 5, 7)["launches"] == 0
    assert lib.sgemm_plan_query(5, 0, 7)["launches"] == 0
    p = lib.sgemm_plan_query(5, 6, 0)
    assert p["launches"] == 1 and p["workspace_bytes"] == 0      # the zero fill
    # M == 0 or N == 0 may pass NULL pointers
    assert lib.sgemm_raw(0, 5, 7, 0, 7, B, 5, 0, 5) == 0
    assert lib.sgemm_raw(5, 0, 7, A, 7, 0, 1, 0, 1) == 0


def test_tile_tables():
    info = lib.sgemm_tile_info("mfma", 0)
    assert info["count"] == 4 and (info["bm"], info["bn"], info["bk"]) == (256, 256, 16)
    for t in range(info["count"]):
        ti = lib.sgemm_tile_info("mfma", t)
        assert ti["bm"] % 32 == 0 and ti["bn"] % 32 == 0 and ti["bk"] % 8 == 0
    assert lib.sgemm_tile_info("valu", 0)["bk"] == 8
    assert lib.sgemm_tile_info("mfma", 99) is None
    assert lib.sgemm_tile_info("naive", 0)["threads"] == 256


def test_boundary_worked_example():
    """The page's edge-handling example: M=300, N=200, K=20 with 128 x 128
    tiles and BK = 8 gives a 3 x 2 grid and 3 K-steps, i.e. the product padded
    to 384 x 256 x 24 ("GEMM from naive to tiled", section 七)."""
    g = json.load(open(os.path.join(GOLDEN, "boundary_example.json")))
    p = lib.sgemm_plan_query(g["M"], g["N"], g["K"], path="valu", tile=0, split_k=1)
    assert (p["bm"], p["bn"], p["bk"]) == (g["BM"], g["BN"], g["BK"])
    assert (p["tiles_m"], p["tiles_n"]) == tuple(g["grid"])
    k_steps = -(-p["k_chunk"] // p["bk"])
    assert k_steps == g["k_steps"]
    assert [p["tiles_m"] * p["bm"], p["tiles_n"] * p["bn"], k_steps * p["bk"]] == g["padded"]


def test_vector_loader_selection():
    # 16-byte aligned, ld and widths multiples of 4 -> 16-byte loaders, nothing packed
    p = lib.sgemm_plan_query(512, 512, 512)
    assert p["vector"] == 1 and p["packed"] == 0 and p["k_padded"] == 512
    # odd leading dimensions (the ragged workload) without packing -> 4-byte loaders
    p = lib.sgemm_plan_query(4097, 3001, 2049, lda=2049, ldb=3001, ldc=3001, pack="never")
    assert p["vector"] == 0 and p["packed"] == 0
    # a base pointer offset by one float
    assert lib.sgemm_plan_query(512, 512, 512, A=0x100004, pack="never")["vector"] == 0
    # forced off: no packing either
    p = lib.sgemm_plan_query(512, 512, 512, A=0x100004, vector=1, pack="always")
    assert p["vector"] == 0 and p["packed"] == 0


def test_packing_plans():
    """Packed operands: which ones, K padded to a multiple of 4, the copies
    at the front of the workspace, one packing launch for both operands."""
    M, N, K = 4097, 3001, 2049
    p = lib.sgemm_plan_query(M, N, K, lda=K, ldb=N, ldc=N, path="mfma", tile=0, decomposition="tiles",
                             split_k=1, pack="always")
    assert p["packed"] == 3 and p["vector"] == 1 and p["k_padded"] == 2052
    # copies with rows padded to 128 bytes: A 4097 x 2080, B 2052 x 3008
    r256 = lambda b: (b + 255) // 256 * 256
    assert p["workspace_bytes"] == r256(M * 2080 * 4) + r256(2052 * 3008 * 4)
    assert p["launches"] == 2
    # only B misaligned (N odd, K a multiple of 4): A is read in place
    q = lib.sgemm_plan_query(512, 509, 512, path="mfma", tile=0, decomposition="tiles", split_k=1,
                             pack="always")
    assert q["packed"] == 2 and q["k_padded"] == 512 and q["workspace_bytes"] == 512 * 512 * 4
    # only A misaligned (odd lda)
    q = lib.sgemm_plan_query(512, 512, 512, lda=513, path="mfma", tile=0, decomposition="tiles", split_k=1,
                             pack="always")
    assert q["packed"] == 1 and q["workspace_bytes"] == 512 * 512 * 4 and q["launches"] == 2
    # aligned operands are never packed; other paths never pack
    assert lib.sgemm_plan_query(512, 512, 512, pack="always")["packed"] == 0
    assert lib.sgemm_plan_query(512, 509, 512, path="valu", pack="always")["packed"] == 0
    with pytest.raises(lib.SgemmError):
        lib.sgemm_plan_query(512, 512, 512, pack=3)


def test_default_plans_fill_the_chip():
    """Every matrix-core benchmark shape gets at least one workgroup per CU
    (256), with split-K or stream-K where the output alone has too few tiles;
    the skinny streaming kernel fills the CUs: K slices in whole rounds of
    one workgroup per CU, or stream-K over two workgroups per CU."""
    shapes = [(4096, 4096, 4096), (4097, 3001, 2049), (8192, 11008, 4096), (16, 11008, 4096),
              (512, 512, 65536)]
    for M, N, K in shapes:
        p = lib.sgemm_plan_query(M, N, K, lda=K, ldb=N, ldc=N)
        if p["path_name"] == "skinny":
            assert p["workgroups"] in ((256, 512) if p["decomposition_name"] == "stream_k" else (256,)), (M, N, K, p)
        else:
            assert p["workgroups"] >= 256, (M, N, K, p)
        Kg = p["k_padded"]
        assert Kg in (K, (K + 3) // 4 * 4)
        assert p["k_chunk"] * p["split_k"] >= Kg
        assert p["k_chunk"] * (p["split_k"] - 1) < Kg
        if p["split_k"] > 1:
            assert p["workspace_bytes"] >= p["split_k"] * M * N * 4
            assert p["launches"] == 2 + (p["packed"] != 0)
        assert lib.sgemm_workspace_size(M, N, K) == p["workspace_bytes"]
    assert lib.sgemm_plan_query(16, 11008, 4096)["path_name"] == "skinny"
    p32 = lib.sgemm_plan_query(32, 11008, 4096)
    assert p32["path_name"] == "skinny" and p32["bm"] == 32
    assert lib.sgemm_plan_query(33, 11008, 4096)["path_name"] == "mfma"
    p = lib.sgemm_plan_query(512, 512, 65536)
    assert p["split_k"] > 1 or p["decomposition_name"] == "stream_k"   # long K is shared out


def test_forced_split_k_slices_cover_k():
    for S in (1, 2, 3, 7, 16):
        p = lib.sgemm_plan_query(300, 200, 1000, path="mfma", tile=2, split_k=S, decomposition="tiles")
        assert p["k_chunk"] % p["bk"] == 0
        assert p["split_k"] <= S
        assert (p["split_k"] - 1) * p["k_chunk"] < 1000 <= p["split_k"] * p["k_chunk"]


def test_stream_k_plans():
    """Stream-K on the 256 x 256 tile: all but the last full wave of tiles are
    data-parallel, the rest is cut into equal K-step ranges, one per CU."""
    p = lib.sgemm_plan_query(8192, 11008, 4096, path="mfma", tile=0, decomposition="stream_k")
    tiles = p["tiles_m"] * p["tiles_n"]
    assert (p["tiles_m"], p["tiles_n"]) == (32, 43) and tiles == 1376
    assert p["decomposition_name"] == "stream_k" and p["workgroups"] == 256
    assert p["dp_tiles"] == 4 * 256 and p["sk_tiles"] == tiles - 4 * 256
    k_steps = 4096 // p["bk"]
    assert p["sk_units_per_wg"] == -(-p["sk_tiles"] * k_steps // 256)
    assert p["launches"] == 2 and p["workspace_bytes"] == 2 * 256 * 256 * 256 * 4
    # whole tiles per workgroup: no partial tiles, no fix-up
    q = lib.sgemm_plan_query(4608, 4608, 32, path="mfma", tile=0, decomposition="stream_k")
    assert q["sk_tiles"] == 324 and q["launches"] == 1 and q["workspace_bytes"] == 0 or \
        q["sk_units_per_wg"] % (32 // q["bk"]) != 0
    # stream-K is for the MFMA path without split-K
    with pytest.raises(lib.SgemmError):
        lib.sgemm_plan_query(512, 512, 512, path="valu", decomposition="stream_k")
    with pytest.raises(lib.SgemmError):
        lib.sgemm_plan_query(512, 512, 512, path="mfma", split_k=2, decomposition="stream_k")


def test_plan_cache_keys():
    """Plans are cached per key: repeated queries agree, and every input the
    plan depends on (operand alignment, leading dimensions, layouts, whether
    A and B are read, options) still changes it after a cached query."""
    M, N, K = 1000, 900, 1200
    first = lib.sgemm_plan_query(M, N, K)
    for _ in range(3):
        assert lib.sgemm_plan_query(M, N, K) == first
    assert first["vector"] == 1 and first["packed"] == 0
    # A 4 bytes off a 16-byte boundary: no 16-byte lanes on A as stored
    mis = lib.sgemm_plan_query(M, N, K, A=0x100004)
    assert mis["vector"] == 0 or mis["packed"] & 1
    # odd leading dimension of B
    odd = lib.sgemm_plan_query(M, N, K, ldb=N + 1)
    assert odd["vector"] == 0 or odd["packed"] & 2
    assert lib.sgemm_plan_query(M, N, K) == first              # the aligned plan is unchanged
    # forced options are part of the key
    forced = lib.sgemm_plan_query(M, N, K, path="mfma", tile=2, split_k=3, decomposition="tiles")
    assert (forced["tile"], forced["split_k"], forced["decomposition_name"]) == (2, 3, "tiles")
    assert lib.sgemm_plan_query(M, N, K, path="valu")["path_name"] == "valu"
    assert lib.sgemm_plan_query(M, N, K) == first
    # layouts and alpha == 0 (no matrix kernel: one scaling launch)
    t = lib.gemm_plan_query("T", "N", M, N, K)
    assert t["path_name"] == "mfma" and 0 <= t["tile"] < lib.sgemm_tile_info("mfma", 0)["count"]
    z = lib.gemm_plan_query("N", "N", M, N, K, alpha=0.0, beta=2.0)
    assert z["launches"] == 1 and z["workspace_bytes"] == 0
    assert lib.gemm_plan_query("N", "N", M, N, K) == first


def test_skinny_plan_rule():
    """The skinny planner: a uniform K split when strips x slices fill the
    256 CUs in whole rounds with at most a quarter of a round idle, else
    stream-K over two workgroups per CU (one with two row blocks)."""
    for M, N, K, split in [(16, 4096, 4096, 4), (1, 4096, 11008, 4), (32, 4096, 11008, 4), (16, 2048, 8192, 8),
                           (16, 8192, 4096, 2), (16, 12800, 4096, 1), (16, 14336, 4096, 1), (4, 1024, 16384, 16),
                           (16, 256, 65536, 64)]:
        p = lib.sgemm_plan_query(M, N, K)
        assert p["path_name"] == "skinny" and p["decomposition_name"] == "tiles", (M, N, K, p)
        assert p["split_k"] == split and p["workgroups"] == -(-N // 64) * split, (M, N, K, p)
    for M, N, K, grid in [(16, 11008, 4096, 512), (8, 11008, 4096, 512), (16, 11008, 8192, 512),
                          (32, 11008, 4096, 256), (16, 22016, 4096, 512), (16, 256, 128, 8)]:
        p = lib.sgemm_plan_query(M, N, K)
        assert p["path_name"] == "skinny" and p["decomposition_name"] == "stream_k", (M, N, K, p)
        assert p["split_k"] == 1 and p["workgroups"] == grid, (M, N, K, p)
    # slices keep at least four 64-deep steps: 4 strips x 2 slices of 256 fill nothing, stream-K it is
    assert lib.sgemm_plan_query(16, 256, 512)["decomposition_name"] == "stream_k"


@pytest.mark.parametrize("shape,tile,decomposition,split", [
    # (timed warm on MI355X: the fastest candidates, microseconds)
    ((424, 384, 744), 3, "tiles", ">1"),       # 64x64 split 4: 11.1, split 2: 12.8, unsplit 15.7
    ((508, 432, 1600), 3, "tiles", ">1"),      # 64x64 split 4: 14.8, 128x128 stream-K: 24.0
    ((528, 448, 832), 3, "tiles", ">1"),       # 64x64 split 4: 12.1, unsplit 16.7
    ((7380, 1184, 340), 3, "tiles", 1),        # 64x64: 64.3, 128x128 stream-K: 77.1
    ((2468, 2160, 440), 3, "tiles", 1),        # 64x64: 52.0, 128x128 stream-K: 60.6
    ((296, 7700, 7252), 3, "tiles", ">1"),     # 64x64 split 2: 299.0, 64x64 stream-K: 338.8
    ((960, 700, 41032), 2, "stream_k", 1),     # 128x128 stream-K: 471.1, 64x64 stream-K: 571.0 (read-bound)
    ((512, 512, 65536), 2, "stream_k", 1),     # 128x128 stream-K: 253.0, split 16: 264.4
])
def test_planner_calibrated_choices(shape, tile, decomposition, split):
    """Plans the fitted time model must keep: shapes where the earlier
    constants chose a candidate 8-59 % slower than the fastest timed one, and
    the long-K workload."""
    p = lib.sgemm_plan_query(*shape, row_tail="never")
    assert (p["tile"], p["decomposition_name"]) == (tile, decomposition), (shape, p)
    assert p["split_k"] > 1 if split == ">1" else p["split_k"] == split, (shape, p)


def test_binding_rejects_overlapping_rows():
    """The binding passes a view's row stride as the leading dimension and
    never widens it: broadcast views (stride 0) and as_strided views whose
    rows overlap are refused before the C call; row- and column-major views
    with padding give their stride."""
    lay = lib._storage_layout
    assert lay((4, 8), (8, 1), "A") == (0, 8)
    assert lay((4, 8), (11, 1), "A") == (0, 11)              # padded rows
    assert lay((1, 8), (0, 1), "A") == (0, 8)                # one row: any stride
    assert lay((4, 1), (1, 1), "A") == (0, 1)                # one column
    for shape, strides in [((4, 8), (0, 1)),                 # expand() of one row
                           ((4, 8), (4, 1)),                 # as_strided rows sharing elements
                           ((4, 1), (0, 1))]:                # broadcast column
        with pytest.raises(ValueError):
            lay(shape, strides, "A")
    # column-major views: only where the operand may be transposed
    assert lay((8, 4), (1, 8), "B", allow_column_major=True) == (1, 8)      # W.t() of an 4 x 8 W
    assert lay((8, 4), (1, 9), "B", allow_column_major=True) == (1, 9)
    with pytest.raises(ValueError):
        lay((8, 4), (1, 4), "B", allow_column_major=True)                 # columns overlap
    with pytest.raises(ValueError):
        lay((8, 4), (1, 8), "C")                                          # C is row-major only
    with pytest.raises(ValueError):
        lay((8, 4), (2, 16), "B", allow_column_major=True)                # neither stride is 1


def test_noalloc_checks_run_before_any_hip_call():
    """sgemm_gemm_noalloc validates and plans on the host before touching the
    device: invalid arguments, a caller workspace, and a forced plan whose
    scratch exceeds the static buffer are refused with no GPU present."""
    o = lib._options
    assert lib.gemm_noalloc_raw(0, 0, -1, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4) == 1         # negative size
    assert lib.gemm_noalloc_raw(2, 0, 4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4) == 1          # bad op flag
    assert lib.gemm_noalloc_raw(0, 0, 64, 64, 64, 1.0, A, 64, B, 64, 0.0, C, 64,
                                opts=o(workspace=0x7000000, workspace_bytes=1 << 20)) == 1
    big = (0, 0, 4096, 4096, 512, 1.0, A, 512, B, 4096, 0.0, C, 4096)
    forced = {"path": "mfma", "tile": 2, "decomposition": "tiles", "split_k": 8}
    assert lib.gemm_plan_query(0, 0, 4096, 4096, 512, **forced)["workspace_bytes"] > lib.NOALLOC_SCRATCH_BYTES
    assert lib.gemm_noalloc_raw(*big, opts=o(**forced)) == 5                                # SGEMM_ERR_SCRATCH_LIMIT
    assert lib.gemm_noalloc_raw(*big, opts=o(path="skinny")) == 1                           # M > 32
    assert "static buffer" in lib.sgemm_status_string(5)
    # empty products enqueue nothing and need no device
    assert lib.gemm_noalloc_raw(0, 0, 0, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4) == 0


def test_read_probe_rejects_bad_arguments():
    """The read-rate probe validates on the host before any HIP call: n a
    multiple of 4, x 16-byte aligned, a partial buffer given."""
    so = lib.load_library()
    assert lib.READ_PROBE_PARTIALS == 4096
    assert lib.read_probe_raw(0x1000, 6, 0x2000) == 1          # n % 4
    assert lib.read_probe_raw(0x1004, 8, 0x2000) == 1          # misaligned x
    assert lib.read_probe_raw(0x1000, -4, 0x2000) == 1         # negative n
    assert lib.read_probe_raw(0x1000, 8, None) == 1            # no partial buffer
    assert lib.read_probe_raw(None, 8, 0x2000) == 1            # no x
    assert so.sgemm_read_probe is not None


def test_fma_probe_rejects_bad_arguments():
    so = lib.load_library()
    assert lib.FMA_PROBE_FMAS_PER_ITER == 128
    assert so.sgemm_fma_probe(-1, 4, 0x1000, None) == 1
    assert so.sgemm_fma_probe(4, 0, 0x1000, None) == 1
    assert so.sgemm_fma_probe(4, 4, None, None) == 1


def test_row_tail_plans():
    """The row tail: M 1-32 rows past a multiple of 64, in every operand
    layout; the main kernel's tiles cover the rows above it."""
    p = lib.sgemm_plan_query(4097, 3001, 2049, lda=2049, ldb=3001, ldc=3001)
    assert p["tail_rows"] == 1 and p["tiles_m"] == 4096 // p["bm"] and p["packed"] == 3
    q = lib.sgemm_plan_query(4097, 3001, 2049, lda=2049, ldb=3001, ldc=3001, row_tail="never")
    assert q["tail_rows"] == 0 and q["tiles_m"] == -(-4097 // q["bm"])
    assert lib.sgemm_plan_query(513, 385, 272, row_tail="always")["tail_rows"] == 1
    assert lib.sgemm_plan_query(4128, 4096, 4096, row_tail="always")["tail_rows"] == 32
    for M in (4096, 4129, 4160, 63, 100):          # none, 33 rows, a multiple, too few rows above
        assert lib.sgemm_plan_query(M, 512, 512, row_tail="always")["tail_rows"] == 0, M
    for ops in [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]:
        q = lib.gemm_plan_query(*ops, 4097, 512, 512, row_tail="always")
        assert q["tail_rows"] == 1 and q["tiles_m"] == 4096 // q["bm"], (ops, q)
    with pytest.raises(lib.SgemmError):
        lib.sgemm_plan_query(4097, 512, 512, row_tail=3)


def test_long_leading_dimensions():
    """The matrix-core loads address each lane by a 32-bit byte offset from
    its tile's first element, so a tile runs only where the farthest element
    of its K-step is within 2^32 bytes: (R - 1) * ld + 15 floats for a
    k-contiguous operand with R rows, 15 * ld + R - 1 for a k-major one.
    Longer strides take a smaller tile, packed copies (which shorten the
    stride), or, when even those are too long, the vector-ALU kernel
    (operands as stored) or the one-thread-per-output kernel."""
    lim = (1 << 30) - 4

    def fits(rows, ld):          # k-contiguous operand of a tile with `rows` rows
        return (rows - 1) * ld + 15 <= lim

    ld = 5_000_000               # too long for the 256-row tiles, not for the 128-row one
    assert not fits(256, ld) and fits(128, ld)
    p = lib.gemm_plan_query("N", "N", 300, 64, 48, lda=ld)
    assert p["path_name"] == "mfma" and p["tile"] in (2, 3) and p["packed"] == 0, p
    for tile in (0, 1):
        with pytest.raises(lib.SgemmError):
            lib.gemm_plan_query("N", "N", 300, 64, 48, lda=ld, path="mfma", tile=tile, pack="never")
        q = lib.gemm_plan_query("N", "N", 300, 64, 48, lda=ld, path="mfma", tile=tile)
        assert q["tile"] == tile and q["packed"] & 1, q          # the packed copy's stride fits
    ld = 20_000_000              # too long for every tile: A is packed (its copy's stride is 64)
    assert not fits(64, ld)
    p = lib.gemm_plan_query("N", "N", 40, 64, 48, lda=ld)
    assert p["path_name"] == "mfma" and p["packed"] == 1, p
    p = lib.gemm_plan_query("N", "N", 64, 64, 16, ldb=72_000_000)   # k-major B: 15 * ldb > 2^30
    assert p["path_name"] == "mfma" and p["packed"] == 2, p
    p = lib.gemm_plan_query("T", "N", 64, 64, 16, lda=72_000_000)   # k-major A
    assert p["path_name"] == "mfma" and p["packed"] == 1, p
    # K itself too long for any tile's rows, packed or not
    K = 17_100_000
    assert not fits(64, K)
    assert lib.gemm_plan_query("N", "N", 33, 4, K)["path_name"] == "valu"
    assert lib.gemm_plan_query("N", "T", 33, 4, K)["path_name"] == "naive"
    with pytest.raises(lib.SgemmError):
        lib.gemm_plan_query("N", "N", 33, 4, K, path="mfma")
    # the skinny path does not use these loads
    assert lib.gemm_plan_query("N", "N", 32, 4, K)["path_name"] == "skinny"


def test_planned_tiles_fit_their_load_offsets():
    """Across random shapes, layouts and long leading dimensions, every
    matrix-core plan (main rows, after packing) uses a tile whose K-step lies
    within the loads' 32-bit byte offsets, restated from the rule."""
    import random
    rng = random.Random(20261203)
    info = [lib.sgemm_tile_info("mfma", t) for t in range(lib.sgemm_tile_info("mfma", 0)["count"])]
    lim = (1 << 30) - 4

    def fits(kc, extent, bk, ld):
        return (extent - 1) * ld + bk - 1 <= lim if kc else (bk - 1) * ld + extent - 1 <= lim

    checked = restricted = 0
    for _ in range(400):
        M, N, K = rng.randint(33, 5000), rng.randint(1, 5000), rng.randint(1, 3000)
        ta, tb = rng.random() < 0.5, rng.random() < 0.5
        a_cols, b_cols = (M if ta else K), (K if tb else N)
        lda = a_cols + rng.choice([0, 1, 7, rng.randint(0, 30_000_000)])
        ldb = b_cols + rng.choice([0, 3, rng.randint(0, 90_000_000)])
        # stand-in addresses far enough apart that these long strides do not make C overlap A or B
        p = lib.gemm_plan_query("T" if ta else "N", "T" if tb else "N", M, N, K, lda=lda, ldb=ldb,
                                A=1 << 20, B=1 << 42, C=1 << 45)
        if p["path_name"] != "mfma":
            continue
        t = info[p["tile"]]
        kp = p["k_padded"]
        # the stride the kernel reads each operand with: a packed copy's rows are padded to 32 floats
        la = -(-((-(-M // 4) * 4) if ta else kp) // 32) * 32 if p["packed"] & 1 else lda
        lb = -(-(kp if tb else (-(-N // 4) * 4)) // 32) * 32 if p["packed"] & 2 else ldb
        assert fits(not ta, t["bm"], t["bk"], la) and fits(tb, t["bn"], t["bk"], lb), (M, N, K, ta, tb, lda, ldb, p)
        checked += 1
        # the stride as stored would not fit the 256 x 256 tiles
        restricted += not (fits(not ta, 256, 16, lda) and fits(tb, 256, 16, ldb))
    assert checked > 200 and restricted > 50, (checked, restricted)
