"""The tiled kernels' index arithmetic, modelled on the host and pinned to
the oracle on small-integer inputs (no GPU).

"如何让计算受限问题真正达到计算受限" (attain.fans), section 5.1, writes the
tiled product as nested loops: output blocks, then the sub-blocks one level
down reuses, then the registers of one thread, with K innermost; the indices
of an output element compose from the levels' offsets.  The models below
walk the same levels with the library's own tile shapes and work
decompositions (read from its host-side plan queries) and sum the products
exactly (integers), so the result must equal the oracle bit for bit and
every output element and every (tile, K-step) unit must be produced exactly
once -- a dropped, repeated or misplaced index fails.
"""
import numpy as np
import pytest

import dense_fp32_matrix_amd as lib
import workloads


def ints(rows, cols, seed):
    return workloads.draw(rows, cols, "integer", seed).numpy()


def mfma_lane_element(lane, reg):
    """Row and column of a 32 x 32 block that lane `lane`, accumulator
    register `reg` of v_mfma_f32_32x32x2_f32 holds."""
    return 8 * (reg // 4) + 4 * (lane // 32) + reg % 4, lane % 32


def test_mfma_output_layout_covers_the_block_once():
    seen = np.zeros((32, 32), dtype=int)
    for lane in range(64):
        for reg in range(16):
            i, j = mfma_lane_element(lane, reg)
            seen[i, j] += 1
    assert np.all(seen == 1)


def blocked_product(A, B, bm, bn, wm, wn):
    """C = A.B walked as the matrix-core kernel tiles it: blocks of bm x bn,
    each split into wave tiles of wm x wn, each into 32 x 32 MFMA blocks whose
    elements belong to (lane, register); per element the K sum runs over the
    K range in ascending order.  Exact (int64); returns C and how often each
    element was written (edges masked as the epilogue masks them)."""
    M, K = A.shape
    N = B.shape[1]
    C = np.zeros((M, N), dtype=np.int64)
    writes = np.zeros((M, N), dtype=int)
    Ai = A.astype(np.int64)
    Bi = B.astype(np.int64)
    for m0 in range(0, M, bm):                                  # output block
        for n0 in range(0, N, bn):
            for w0 in range(0, bm, wm):                         # wave tile
                for v0 in range(0, bn, wn):
                    for b0 in range(0, wm, 32):                 # 32 x 32 MFMA block
                        for c0 in range(0, wn, 32):
                            for lane in range(64):              # lane, register
                                for reg in range(16):
                                    di, dj = mfma_lane_element(lane, reg)
                                    i = m0 + w0 + b0 + di
                                    j = n0 + v0 + c0 + dj
                                    if i < M and j < N:          # the epilogue's mask
                                        C[i, j] = int(np.dot(Ai[i, :], Bi[:, j]))
                                        writes[i, j] += 1
    return C, writes


@pytest.mark.parametrize("tile", [2, 3])
def test_blocked_walk_matches_oracle(oracle_mod, tile):
    """The 128 x 128 (8 waves of 64 x 32) and 64 x 64 (4 waves of 32 x 32)
    tiles over a ragged product spanning several blocks."""
    info = lib.sgemm_tile_info("mfma", tile)
    bm, bn = info["bm"], info["bn"]
    waves = info["threads"] // 64
    wm, wn = (64, 32) if waves == 8 else (32, 32)
    assert (bm // wm) * (bn // wn) == waves
    M, N, K = bm + 37, 2 * bn - 5, 23
    A, B = ints(M, K, 1), ints(K, N, 2)
    C, writes = blocked_product(A, B, bm, bn, wm, wn)
    assert np.all(writes == 1)
    assert np.array_equal(C.astype(np.float64), oracle_mod.sgemm(A, B))


def stream_k_items(plan, K):
    """The work items of the stream-K decomposition, as the kernel walks them
    for every persistent workgroup: first data-parallel tiles t = w, w + P,
    ..., each over all K-steps; then the workgroup's range of (tile, K-step)
    units, cut at tile boundaries.  Yields (workgroup, slot or None, tile,
    first K-step, end K-step)."""
    P, dp, ipw = plan["workgroups"], plan["dp_tiles"], plan["sk_units_per_wg"]
    ks = -(-K // plan["bk"])
    units = plan["sk_tiles"] * ks
    for w in range(P):
        for t in range(w, dp, P):
            yield w, None, t, 0, ks
        it, end, which = w * ipw, min((w + 1) * ipw, units), 0
        while it < end:
            j, q0 = divmod(it, ks)
            q1 = min(ks, q0 + (end - it))
            yield w, (None if (q0 == 0 and q1 == ks) else which), dp + j, q0, q1
            which = 1
            it += q1 - q0


@pytest.mark.parametrize("tile", [0, 2, 3])
@pytest.mark.parametrize("shape", [(300, 200, 1000), (1000, 700, 160), (4352, 4352, 48)],
                         ids=lambda s: "x".join(map(str, s)))
def test_stream_k_schedule(oracle_mod, tile, shape):
    """The planner's stream-K numbers (grid, data-parallel tiles, units per
    workgroup) give every (tile, K-step) to exactly one workgroup; summing
    each tile's partial slots in workgroup order, as the fix-up does, gives
    the oracle's product (checked on a 4352 x 4352 plan by coverage only)."""
    M, N, K = shape
    plan = lib.sgemm_plan_query(M, N, K, path="mfma", tile=tile, decomposition="stream_k")
    bm, bn, bk = plan["bm"], plan["bn"], plan["bk"]
    tiles = plan["tiles_m"] * plan["tiles_n"]
    ks = -(-K // bk)
    assert plan["dp_tiles"] + plan["sk_tiles"] == tiles
    cover = np.zeros((tiles, ks), dtype=int)
    items = list(stream_k_items(plan, K))
    for w, slot, t, q0, q1 in items:
        cover[t, q0:q1] += 1
    assert np.all(cover == 1)
    # the plan needs a fix-up (and workspace) exactly when some range cuts a tile
    cut = any(slot is not None for _, slot, _, _, _ in items)
    assert (plan["launches"] == 2) == cut and (plan["workspace_bytes"] > 0) == cut
    if M * N * K > 2e8:
        return
    A, B = ints(M, K, 3), ints(K, N, 4)
    Ai, Bi = A.astype(np.int64), B.astype(np.int64)
    C = np.zeros((M, N), dtype=np.int64)
    partial = {}
    for w, slot, t, q0, q1 in items:
        tm, tn = divmod(t, plan["tiles_n"])         # any bijection; the kernel's is checked elsewhere
        r0, c0 = tm * bm, tn * bn
        k0, k1 = q0 * bk, min(K, q1 * bk)
        p = Ai[r0:r0 + bm, k0:k1] @ Bi[k0:k1, c0:c0 + bn]
        if slot is None:
            C[r0:r0 + bm, c0:c0 + bn] = p
        else:
            partial.setdefault(t, []).append((w, p))
    for t, parts in partial.items():
        tm, tn = divmod(t, plan["tiles_n"])
        ws = [w for w, _ in parts]
        assert ws == sorted(ws) and len(ws) >= 2      # contributors in workgroup order
        C[tm * bm:(tm + 1) * bm, tn * bn:(tn + 1) * bn] = sum(p for _, p in parts)
    assert np.array_equal(C.astype(np.float64), oracle_mod.sgemm(A, B))


@pytest.mark.parametrize("path,tile", [("mfma", 2), ("mfma", 3), ("valu", 0), ("skinny", 0)])
@pytest.mark.parametrize("split", [2, 3, 7])
def test_split_k_slices(oracle_mod, path, tile, split):
    """Split-K: the plan's K chunk cuts K into slices that cover it once;
    the slices' partial products, summed in slice order, give the oracle's."""
    M, N, K = (16, 300, 1000) if path == "skinny" else (150, 170, 1000)
    plan = lib.sgemm_plan_query(M, N, K, path=path, tile=tile, split_k=split, decomposition="tiles")
    S, kc = plan["split_k"], plan["k_chunk"]
    assert kc % plan["bk"] == 0 and (S - 1) * kc < K <= S * kc
    A, B = ints(M, K, 5), ints(K, N, 6)
    Ai, Bi = A.astype(np.int64), B.astype(np.int64)
    C = sum(Ai[:, z * kc:min(K, (z + 1) * kc)] @ Bi[z * kc:min(K, (z + 1) * kc), :] for z in range(S))
    assert np.array_equal(C.astype(np.float64), oracle_mod.sgemm(A, B))
