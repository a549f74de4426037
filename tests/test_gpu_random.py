"""GPU parity on seeded random problems of the library-call form
C = alpha * op(A) op(B) + beta * C ("GEMM from naive to tiled", section 二.2;
alpha and beta as in the epilogue of section 九.2), against the oracle's gemm.

Each case draws its sizes (1 to 700, log-uniform, some below 17, a fifth
with M a few rows past a multiple of 64), the two operation flags, the leading dimensions of A, B and C (padding filled with
NaN), alpha and beta.  Half the cases run the library's own plan, so the
planner's choices on shapes no fixed case names are checked; the other half
force a plan drawn at random among those the library accepts (tile, work
decomposition, K slices, packing, row tail, or the skinny path), pairings
the fixed cases do not make.

Bar (tests/checks.py): |C - C_ref| <= 1e-5 * D elementwise with
D = |alpha| sum_k |op(A)||op(B)| + |beta| |C_in|; bit-exact on small-integer
inputs, with alpha in {1, 2, -0.75} and beta in {0, 0.5, -1}, where every
step is exact in FP32.
"""
import math
import random

import pytest
import torch

import dense_fp32_matrix_amd as lib
import workloads
from checks import assert_bit_exact, assert_within_bound

DEV = "cuda:0"
CASES = 400


def say(msg):
    print(f"[case] {msg}", flush=True)


def _size(rng):
    if rng.random() < 0.15:
        return rng.randint(1, 16)
    return int(round(math.exp(rng.uniform(math.log(17), math.log(700)))))


def _pad(rng):
    return rng.choice([0, 0, 0, 1, 3, 4, 17])


def _forced_plan(rng, M, N, K, ta, tb, lda, ldb, ldc):
    """A plan drawn at random among the ones the library accepts here."""
    for _ in range(50):
        if M <= 32 and rng.random() < 0.3:
            o = {"path": "skinny", "decomposition": rng.choice(["tiles", "stream_k"])}
            if o["decomposition"] == "tiles":
                o["split_k"] = rng.choice([1, 2, 3])
        else:
            o = {"path": "mfma", "tile": rng.randrange(lib.sgemm_tile_info("mfma", 0)["count"]),
                 "decomposition": rng.choice(["tiles", "stream_k"]),
                 "pack": rng.choice(["auto", "never", "always"]),
                 "row_tail": rng.choice(["auto", "never", "always"])}
            if o["decomposition"] == "tiles":
                o["split_k"] = rng.choice([1, 2, 3, 5])
        try:
            lib.gemm_plan_query("T" if ta else "N", "T" if tb else "N", M, N, K, alpha=1.0, lda=lda, ldb=ldb,
                                ldc=ldc, **o)
            return o
        except lib.SgemmError:
            continue
    return {}


def _case(i):
    rng = random.Random(7919 * (i + 1))
    M, N, K = _size(rng), _size(rng), _size(rng)
    ta, tb = rng.random() < 0.5, rng.random() < 0.5
    if rng.random() < 0.2:
        # a few rows past a multiple of 64, operands as stored: the row tail's case
        M, ta, tb = 64 * rng.randint(1, 8) + rng.randint(1, 32), False, False
    a_rows, a_cols = (K, M) if ta else (M, K)
    b_rows, b_cols = (N, K) if tb else (K, N)
    lda, ldb, ldc = a_cols + _pad(rng), b_cols + _pad(rng), N + _pad(rng)
    alpha = rng.choice([1.0, 2.0, -0.75])
    beta = rng.choice([0.0, 0.5, -1.0])
    opts = _forced_plan(rng, M, N, K, ta, tb, lda, ldb, ldc) if i % 2 else {}
    return dict(M=M, N=N, K=K, ta=ta, tb=tb, a_shape=(a_rows, a_cols), b_shape=(b_rows, b_cols), lda=lda,
                ldb=ldb, ldc=ldc, alpha=alpha, beta=beta, opts=opts, seed=1000 + 11 * i)


def _to_dev(x, ld):
    """Device copy of the (rows, cols) CPU tensor x with row stride ld (NaN in the gap)."""
    rows, cols = x.shape
    buf = torch.full((max(rows, 1), ld), float("nan"), dtype=torch.float32)
    buf[:rows, :cols] = x
    return buf.to(DEV)[:rows, :cols]


def _run(c, kind):
    A = workloads.draw(*c["a_shape"], kind, c["seed"])
    B = workloads.draw(*c["b_shape"], kind, c["seed"] + 1)
    Cin = workloads.draw(c["M"], c["N"], kind, c["seed"] + 2)
    Ad, Bd = _to_dev(A, c["lda"]), _to_dev(B, c["ldb"])
    Cd = _to_dev(Cin, c["ldc"]) if c["beta"] != 0 else \
        torch.full((c["M"], c["ldc"]), float("nan"), device=DEV)[:, :c["N"]]
    lib.gemm(Ad, Bd, Cd, trans_a=c["ta"], trans_b=c["tb"], alpha=c["alpha"], beta=c["beta"], **c["opts"])
    torch.cuda.synchronize()
    return A, B, Cin, Cd.cpu().numpy()


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(CASES))
def test_random_problem(oracle_mod, i):
    c = _case(i)
    what = (f"random {i}: M={c['M']} N={c['N']} K={c['K']} ta={c['ta']} tb={c['tb']} lda={c['lda']} "
            f"ldb={c['ldb']} ldc={c['ldc']} alpha={c['alpha']} beta={c['beta']} opts={c['opts']}")
    say(what)
    A, B, Cin, got = _run(c, "uniform")
    ref, D = oracle_mod.gemm(A.numpy(), B.numpy(), Cin.numpy(), trans_a=c["ta"], trans_b=c["tb"],
                             alpha=c["alpha"], beta=c["beta"], with_denominator=True)
    assert_within_bound(got, ref, D, what=what)
    Ai, Bi, Ci, goti = _run(c, "integer")
    refi = oracle_mod.gemm(Ai.numpy(), Bi.numpy(), Ci.numpy(), trans_a=c["ta"], trans_b=c["tb"],
                           alpha=c["alpha"], beta=c["beta"])
    assert_bit_exact(goti, oracle_mod.round_to_f32(refi), what=what + " int")


def test_random_cases_cover_the_plans():
    """The drawn cases reach every matrix-core tile, both decompositions,
    packing, 4-byte lanes and the row tail among the plans they run (checked
    on the host, from the plans the library reports)."""
    seen = set()
    for i in range(CASES):
        c = _case(i)
        p = lib.gemm_plan_query("T" if c["ta"] else "N", "T" if c["tb"] else "N", c["M"], c["N"], c["K"],
                                alpha=c["alpha"], beta=c["beta"], lda=c["lda"], ldb=c["ldb"], ldc=c["ldc"],
                                **c["opts"])
        seen.add(("path", p["path_name"]))
        if p["path_name"] == "mfma":
            seen.add(("tile", p["tile"]))
        seen.add(("decomposition", p["decomposition_name"]))
        seen.add(("packed", p["packed"] != 0))
        seen.add(("vector", p["vector"]))
        seen.add(("tail", p["tail_rows"] > 0))
        seen.add(("split", p["split_k"] > 1))
    need = {("tile", t) for t in range(4)} | {("decomposition", "tiles"), ("decomposition", "stream_k"),
                                            ("packed", True), ("vector", 0), ("tail", True), ("split", True)}
    assert need <= seen, sorted(need - seen)
