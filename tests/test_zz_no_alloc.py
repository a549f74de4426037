"""sgemm_gemm_noalloc -- the entry point that allocates no device memory --
called through the C interface and checked against sgemm_gemm_ex, the entry
point it is a variant of, on the same inputs.

Every case makes two calls in a row on one stream, the second with a smaller
input, so the second runs on the static scratch the first left behind.  The
bar is the parity bar of the other GPU tests: bit-exact on small-integer
inputs (against the oracle and against sgemm_gemm_ex), and within
1e-5 * sum_k |a||b| of the oracle on uniform inputs; where the plan is the
one sgemm_gemm_ex uses (its scratch fits the static buffer) the two entry
points must return the same bits.
"""
import numpy as np
import pytest
import torch

import dense_fp32_matrix_amd as lib
import workloads
from checks import assert_bit_exact, assert_within_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCRATCH_LIMIT = 5          # SGEMM_ERR_SCRATCH_LIMIT
INVALID_ARG = 1


def say(msg):
    print(f"[case] {msg}", flush=True)


def stored(M, N, K, ta, tb, kind, seed, lda=None, ldb=None):
    """Stored A (K x M when ta) and B (N x K when tb), with NaN-padded rows
    when a leading dimension above the width is asked for."""
    A = workloads.draw(K, M, kind, seed) if ta else workloads.draw(M, K, kind, seed)
    B = workloads.draw(N, K, kind, seed + 1) if tb else workloads.draw(K, N, kind, seed + 1)
    A = workloads.with_ld(A, lda or A.shape[1])
    B = workloads.with_ld(B, ldb or B.shape[1])
    return A, B


def to_dev(x):
    """Device copy keeping the row stride (the NaN padding included)."""
    if x.shape[0] > 0 and x.stride(0) != x.shape[1]:
        base = torch.full((x.shape[0], x.stride(0)), float("nan"))
        base[:, :x.shape[1]] = x
        return base.to(DEV)[:, :x.shape[1]]
    return x.contiguous().to(DEV)


def call(noalloc, Ad, Bd, C, ta, tb, alpha, beta, opts):
    """One raw C call; returns the status."""
    M, N = C.shape
    K = Ad.shape[0] if ta else Ad.shape[1]
    fn = lib.gemm_noalloc_raw if noalloc else lib.gemm_raw
    o = lib._options(**opts) if opts is not None else None
    return fn(int(ta), int(tb), M, N, K, alpha, Ad.data_ptr(), Ad.stride(0), Bd.data_ptr(), Bd.stride(0), beta,
              C.data_ptr(), C.stride(0), torch.cuda.current_stream().cuda_stream, o)


def reference(oracle_mod, A, B, ta, tb, alpha, beta, C0, with_d):
    return oracle_mod.gemm(A.numpy(), B.numpy(), C0.numpy() if beta != 0 else None, trans_a=ta, trans_b=tb,
                           alpha=alpha, beta=beta, with_denominator=with_d)


CASES = [
    # (name, opts, [(M, N, K, ta, tb, lda, ldb) first call, second call (smaller)])
    ("stream-K partial tiles, 128x128", {"path": "mfma", "tile": 2, "decomposition": "stream_k"},
     [(1000, 900, 3000, False, False, None, None), (600, 517, 700, False, False, None, None)]),
    ("stream-K after data-parallel tiles, 256x256, X.W^T", {"path": "mfma", "tile": 1, "decomposition": "stream_k"},
     [(5888, 5888, 160, False, True, None, None), (2944, 2944, 96, False, True, None, None)]),
    ("split-K, 64x64", {"path": "mfma", "tile": 3, "decomposition": "tiles", "split_k": 4},
     [(700, 600, 2000, False, False, None, None), (300, 260, 900, False, False, None, None)]),
    ("packed operands, stream-K", {"path": "mfma", "tile": 2, "pack": "always", "decomposition": "stream_k"},
     [(513, 385, 272, False, False, 273, 387), (130, 261, 101, True, False, None, None)]),
    ("skinny stream-K", {"path": "skinny", "decomposition": "stream_k"},
     [(16, 3000, 1000, False, False, None, None), (5, 700, 333, False, False, None, None)]),
    ("skinny split-K", {"path": "skinny", "split_k": 3},
     [(32, 1000, 4100, False, False, None, None), (9, 300, 1000, False, False, None, None)]),
    ("valu split-K", {"path": "valu", "split_k": 5},
     [(300, 200, 2000, False, False, None, None), (130, 100, 700, False, False, None, None)]),
    ("row tail, then packed operands with a row tail", {"row_tail": "always"},
     [(1025, 600, 700, False, False, None, None), (577, 301, 205, False, False, 207, 303)]),
    ("default plan", None,
     [(512, 512, 8192, False, False, None, None), (300, 200, 20, False, False, None, None)]),
    ("default plan, unaligned operands", None,
     [(1001, 777, 515, False, False, 517, 779), (257, 130, 33, False, True, None, None)]),
    # the default plan of sgemm_gemm packs both operands here (205 MiB of
    # scratch); the no-allocation plan is the fastest that fits the static buffer
    ("default plan above the static buffer", None,
     [(6001, 5001, 4097, False, False, 4099, 5003), (2000, 1500, 1000, False, False, 1001, None)]),
]


@pytest.mark.parametrize("kind", ["integer", "uniform"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0].replace(" ", "_"))
def test_noalloc_matches_gemm_ex(oracle_mod, case, kind):
    name, opts, shapes = case
    alpha, beta = (2.0, -0.5) if kind == "integer" else (1.0, 0.0)
    jobs = []
    for i, (M, N, K, ta, tb, lda, ldb) in enumerate(shapes):
        A, B = stored(M, N, K, ta, tb, kind, 900 + 10 * i + M % 7, lda, ldb)
        C0 = workloads.draw(M, N, kind, 950 + i)
        jobs.append((M, N, K, ta, tb, A, B, C0, to_dev(A), to_dev(B)))
    same_plan = []
    for M, N, K, ta, tb, A, B, C0, Ad, Bd in jobs:
        q = lib.gemm_plan_query(int(ta), int(tb), M, N, K, alpha=alpha, A=Ad.data_ptr(), lda=Ad.stride(0),
                                B=Bd.data_ptr(), ldb=Bd.stride(0), beta=beta, **(opts or {}))
        same_plan.append(q["workspace_bytes"] <= lib.NOALLOC_SCRATCH_BYTES)
    if opts is not None:
        assert all(same_plan), "forced plans of these cases fit the static buffer"
    # the existing entry point, one call at a time
    ref_out = []
    for M, N, K, ta, tb, A, B, C0, Ad, Bd in jobs:
        C = C0.to(DEV) if beta != 0 else torch.full((M, N), float("nan"), device=DEV)
        say(f"{name} {kind}: sgemm_gemm_ex {M}x{N}x{K} ta={ta} tb={tb}")
        assert call(False, Ad, Bd, C, ta, tb, alpha, beta, opts) == 0
        torch.cuda.synchronize()
        ref_out.append(C.cpu().numpy())
    # the no-allocation entry point: both calls back to back, then one synchronisation
    outs = []
    for M, N, K, ta, tb, A, B, C0, Ad, Bd in jobs:
        C = C0.to(DEV) if beta != 0 else torch.full((M, N), float("nan"), device=DEV)
        outs.append(C)
    torch.cuda.synchronize()
    for (M, N, K, ta, tb, A, B, C0, Ad, Bd), C in zip(jobs, outs):
        say(f"{name} {kind}: sgemm_gemm_noalloc {M}x{N}x{K} ta={ta} tb={tb}")
        assert call(True, Ad, Bd, C, ta, tb, alpha, beta, opts) == 0
    torch.cuda.synchronize()
    for (M, N, K, ta, tb, A, B, C0, Ad, Bd), C, Cref, same in zip(jobs, outs, ref_out, same_plan):
        got = C.cpu().numpy()
        what = f"{name} {kind} {M}x{N}x{K}"
        if kind == "integer":
            exact = oracle_mod.round_to_f32(reference(oracle_mod, A, B, ta, tb, alpha, beta, C0, False))
            assert_bit_exact(got, exact, what=what + " vs oracle")
            assert_bit_exact(Cref, exact, what=what + " sgemm_gemm_ex vs oracle")
        else:
            val, D = reference(oracle_mod, A, B, ta, tb, alpha, beta, C0, True)
            assert_within_bound(got, val, D, what=what + " vs oracle")
            assert_within_bound(Cref, val, D, what=what + " sgemm_gemm_ex vs oracle")
        if same:
            assert_bit_exact(got, Cref, what=what + " vs sgemm_gemm_ex (same plan)")


def test_noalloc_rejects_what_does_not_fit():
    """A forced plan whose scratch exceeds the static buffer, and a caller
    workspace, are refused before anything is enqueued: C keeps its NaN."""
    M, N, K = 4096, 4096, 512
    Ad = torch.ones((M, K), device=DEV)
    Bd = torch.ones((K, N), device=DEV)
    C = torch.full((M, N), float("nan"), device=DEV)
    torch.cuda.synchronize()
    opts = {"path": "mfma", "tile": 2, "decomposition": "tiles", "split_k": 8}
    assert lib.gemm_plan_query(0, 0, M, N, K, **opts)["workspace_bytes"] > lib.NOALLOC_SCRATCH_BYTES
    say("noalloc over the limit")
    assert call(True, Ad, Bd, C, False, False, 1.0, 0.0, opts) == SCRATCH_LIMIT
    ws = torch.empty(1 << 20, device=DEV)
    assert call(True, Ad, Bd, C, False, False, 1.0, 0.0, {"workspace": ws}) == INVALID_ARG
    torch.cuda.synchronize()
    assert torch.isnan(C).all()
    with pytest.raises(lib.SgemmError):
        lib.gemm_noalloc(Ad, Bd, C, **opts)
    # the same forced plan on the existing entry point is fine
    assert call(False, Ad, Bd, C, False, False, 1.0, 0.0, opts) == 0
    torch.cuda.synchronize()
    assert torch.all(C == K)
