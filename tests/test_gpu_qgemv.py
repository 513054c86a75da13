"""Parity of the fused dequantize-and-multiply with the oracle (GPU).

The oracle forms What exactly as the reconstruction writes it and multiplies
in float64.  The kernel sums in float32, so every output is held to the
bound the header states:
    |Y[b,i] - Y_ref[b,i]| <= (N/32 + nnz_i + 40) * 2^-24 * T[b,i],
    T[b,i] = sum_j |Wd[i,j] x[b,j]| + sum_{salient j} (|Wd[i,j]| + |val|) |x[b,j]|,
with Wd the reconstruction without the sparse overwrite.  The cases cover
one and several column slabs, every token-chunk width (1, 2, 4, 8 and mixes),
the residual codebook in LDS and in global memory, no residual stage, d < 8,
misaligned pointers (scalar path), rows with no / all salient entries, and
B = 0.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, host
from hessian_weighted_vector_amd import vq

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_case(seed, M, N, d, K1, K2, B, scales=True, nnz_per_row=3, full_row=None):
    """Seeded compressed matrix + activations (no method arithmetic)."""
    g = np.random.default_rng([123, seed])
    nb = N // d
    C1 = (0.02 * g.standard_t(4.0, size=(K1, d))).astype(np.float32)
    C2 = (0.004 * g.standard_normal((K2, d))).astype(np.float32) if K2 else None
    i1 = g.integers(0, K1, M * nb).astype(np.uint16)
    i2 = g.integers(0, K2, M * nb).astype(np.uint16) if K2 else None
    r = g.uniform(0.5, 2.0, M).astype(np.float32) if scales else None
    c = g.uniform(0.5, 2.0, N).astype(np.float32) if scales else None
    rp = col = val = None
    if nnz_per_row is not None:
        per = g.integers(0, nnz_per_row + 1, size=M)
        per[0] = 0
        if full_row is not None:
            per[full_row] = N
        rp = np.concatenate([[0], np.cumsum(per)]).astype(np.int32)
        col = np.concatenate([np.sort(g.choice(N, k, replace=False)) for k in per]).astype(np.int32)
        val = (0.2 * g.standard_t(3.0, size=col.size)).astype(np.float32)
    X = g.standard_normal((B, N)).astype(np.float32)
    return dict(M=M, N=N, d=d, C1=C1, idx1=i1, C2=C2, idx2=i2, r=r, c=c, row_ptr=rp, col=col, val=val), X


def reference_and_bound(cs, X):
    Y = oracle.qgemv(X=X, **cs)
    dense = dict(cs, row_ptr=None, col=None, val=None)
    Wd = np.abs(oracle.reconstruct(**dense).astype(np.float64))
    Xa = np.abs(X.astype(np.float64))
    T = Xa @ Wd.T
    M, N = cs["M"], cs["N"]
    nnz_i = np.zeros(M)
    if cs["row_ptr"] is not None:
        rp, col, val = cs["row_ptr"], cs["col"], cs["val"]
        nnz_i = np.diff(rp).astype(np.float64)
        rows = np.repeat(np.arange(M), np.diff(rp))
        w = Wd[rows, col] + np.abs(val.astype(np.float64))
        extra = np.zeros((X.shape[0], M))
        np.add.at(extra.T, rows, (w[:, None] * Xa[:, col].T))
        T = T + extra
    tol = (N / 32.0 + nnz_i[None, :] + 40.0) * U32 * T
    return Y, tol


def run_gpu(cs, X, misalign=False):
    def d_(a):
        return None if a is None else dev(a)
    if misalign:
        # a view one float into a larger buffer: pointers no longer 16-byte aligned
        Xb = torch.zeros(X.size + 1, dtype=torch.float32, device="cuda")
        Xb[1:] = dev(X.ravel())
        Xg = Xb[1:].view(X.shape)
    else:
        Xg = dev(X)
    return vq.qgemv(cs["M"], cs["N"], cs["d"], d_(cs["C1"]), d_(cs["idx1"]), Xg, d_(cs["C2"]), d_(cs["idx2"]),
                    d_(cs["r"]), d_(cs["c"]), d_(cs["row_ptr"]), d_(cs["col"]), d_(cs["val"]))


def check(cs, X, got):
    Y, tol = reference_and_bound(cs, X)
    got = host(got).astype(np.float64)
    err = np.abs(got - Y)
    worst = float((err / np.maximum(tol, 1e-300)).max()) if err.size else 0.0
    say("  max err / bound = %.3g" % worst)
    assert np.all(err <= tol), worst


CASES = [
    # (seed, M, N, d, K1, K2, B, scales, nnz_per_row)
    (1, 64, 64, 8, 16, 0, 1, False, None),
    (2, 37, 40, 8, 33, 5, 3, True, 3),          # ragged rows, chunks 2 + 1
    (3, 130, 256, 8, 256, 256, 8, True, 6),     # residual codebook in LDS (256 x 8 floats)
    (4, 70, 512, 8, 1000, 300, 5, True, 9),     # residual codebook in global memory; chunks 4 + 1
    (5, 16, 24, 3, 7, 4, 2, True, 2),           # d = 3 (scalar path)
    (6, 8, 8, 1, 5, 3, 1, True, 1),             # d = 1
    (7, 50, 96, 6, 40, 0, 13, False, 4),        # d = 6, chunks 8 + 4 + 1
    (8, 33, 30008, 8, 4096, 256, 9, True, 40),  # several column slabs (3 at one token, 17 at eight)
    (9, 9, 200, 5, 11, 7, 4, True, 5),          # d = 5, several salient entries per row
]


@pytest.mark.parametrize("case", CASES, ids=["c%d" % c[0] for c in CASES])
def test_qgemv_matches_oracle(case):
    seed, M, N, d, K1, K2, B, scales, nz = case
    say("qgemv", case)
    cs, X = make_case(seed, M, N, d, K1, K2, B, scales, nz)
    check(cs, X, run_gpu(cs, X))


def test_qgemv_scalar_path_misaligned_and_full_rows():
    say("qgemv misaligned X, one fully salient row")
    cs, X = make_case(21, 40, 128, 8, 64, 32, 3, True, 4, full_row=7)
    got = run_gpu(cs, X, misalign=True)
    check(cs, X, got)
    # and the vector path on the same inputs agrees within the same bound
    check(cs, X, run_gpu(cs, X))


def test_qgemv_reproducible_and_empty():
    say("qgemv reproducibility, B = 0")
    cs, X = make_case(22, 300, 1024, 8, 512, 64, 8, True, 12)
    a = host(run_gpu(cs, X))
    b = host(run_gpu(cs, X))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    X0 = torch.empty((0, cs["N"]), dtype=torch.float32, device="cuda")
    Y0 = vq.qgemv(cs["M"], cs["N"], 8, dev(cs["C1"]), dev(cs["idx1"]), X0)
    assert Y0.shape == (0, cs["M"])


def test_qgemv_unit_tokens_read_columns():
    """e_j as a token gives column j of the reconstruction: exact when no row
    scale rounds (rscale = 1) and no salient entry shares the row, since then
    every product is exact and only one term is non-zero."""
    say("qgemv unit tokens")
    cs, _ = make_case(23, 24, 64, 8, 30, 6, 1, False, None)
    N = cs["N"]
    X = np.eye(N, dtype=np.float32)
    What = oracle.reconstruct(**cs)
    got = host(run_gpu(cs, X))
    assert np.array_equal(got.view(np.uint32), np.ascontiguousarray(What.T).view(np.uint32))
