"""Parity of Algorithm 1 (second-order error propagation, column sub-vectors)
with the oracle (GPU).

The library keeps the working matrix and the errors in float64 and takes
every update in the oracle's order and rounding (VPTQ page, "The Core
Algorithm", Algorithm 1: the in-block update column by column, the block's
end update as one sum over the block's columns), and every nearest-row
decision equals the exact float64 direct-form one (the matrix-core search
certifies its winner against a rounding bound; the rest is searched again
exactly).  So the whole trajectory equals the oracle's bit for bit:
  * indices equal everywhere, with no parting;
  * What equal bit for bit (codebook rows);
  * E (float64 inside, returned as float32) equal to the oracle's float64 E
    rounded to float32, bit for bit.
Cases cover V = 8 (matrix-core path) and V = 4, 6 (vector path), K below, at
and across 256- and 512-centroid chunks, K = 1, blocks that do not divide N,
B > N, B = 1, U = I, an unaligned codebook (direct form for V = 8), working
values 1e-6 and 1e4 times the codebook's scale, an all-zero codebook (every
decision a tie, all of them searched again exactly), and the 4096 x 11008
workload on 32 sampled row groups.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev, host
from hessian_weighted_vector_amd import configs, synth, vq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_case(seed, M, N, V, K, T=64, eye=False):
    g = np.random.default_rng([61, seed])
    W = (0.02 * g.standard_t(4.0, size=(M, N))).astype(np.float32)
    X = g.standard_normal((T, N))
    X[:, g.choice(N, max(1, N // 20), replace=False)] *= 10.0
    U = np.eye(N, dtype=np.float32) if eye else oracle.inverse_hessian_factor(X.T @ X).astype(np.float32)
    cols = W.T.reshape(-1, V)
    if K <= cols.shape[0]:
        C = cols[np.sort(g.choice(cols.shape[0], K, replace=False))].copy()
    else:
        C = (0.02 * g.standard_normal((K, V))).astype(np.float32)
    return W, U, C


def compare(W, U, C, V, B, idx_g, What_g, E_g, rows=None):
    """The GPU trajectory against the oracle run on the same rows (groups of V
    rows evolve independently given U and C): indices, What and E (rounded to
    float32) identical.  Returns the number of row groups compared."""
    Wr = W if rows is None else W[rows]
    idx_o, What_o, E_o, _ = oracle.vptq(Wr, U, V, C, B)
    bad = np.argwhere(idx_g != idx_o)
    assert bad.size == 0, ("index differs at (column, group)", bad[:10])
    assert np.array_equal(What_g.view(np.uint32), What_o.view(np.uint32))
    if E_g is not None:
        assert np.array_equal(E_g.view(np.uint32), E_o.astype(np.float32).view(np.uint32)), \
            float(np.abs(E_g.astype(np.float64) - E_o).max())
    return Wr.shape[0] // V


CASES = [
    # (seed, M, N, V, K, B)
    (1, 64, 96, 8, 32, 16),
    (2, 60, 50, 4, 100, 7),      # scalar path, blocks that do not divide N
    (3, 32, 40, 8, 700, 128),    # three centroid chunks, one block (B > N)
    (4, 16, 24, 8, 1, 5),        # K = 1
    (5, 96, 300, 6, 64, 128),    # V = 6, three blocks, the last ragged
    (6, 40, 20, 8, 256, 1),      # B = 1, exactly one centroid chunk
]


@pytest.mark.parametrize("case", CASES, ids=["v%d" % c[0] for c in CASES])
def test_vptq_matches_oracle(case):
    seed, M, N, V, K, B = case
    say("vptq", case)
    W, U, C = make_case(seed, M, N, V, K)
    idx, What, E = vq.vptq(dev(W), dev(U), V, dev(C), B, want_E=True)
    compare(W, U, C, V, B, host(idx).reshape(N, M // V), host(What), host(E))


def test_vptq_identity_is_plain_column_vq():
    """U = I: no coupling, each column's sub-vectors take their Euclidean nearest
    codebook rows and E = W - What exactly."""
    say("vptq U = I")
    W, U, C = make_case(7, 48, 33, 8, 50, eye=True)
    idx, What, E = vq.vptq(dev(W), dev(U), 8, dev(C), 10, want_E=True)
    compare(W, U, C, 8, 10, host(idx).reshape(33, 6), host(What), host(E))
    assert np.array_equal(host(E), W - host(What))


def test_vptq_reproducible():
    say("vptq reproducibility")
    W, U, C = make_case(8, 64, 200, 8, 300)
    a = [vq.vptq(dev(W), dev(U), 8, dev(C), 32, want_E=True) for _ in range(2)]
    for x, y in zip(a[0], a[1]):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.uint16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.uint16 else y.view(torch.int32))


def test_vptq_unaligned_codebook_takes_the_direct_form():
    """V = 8 with a codebook that is not 16-byte aligned runs the direct-form
    search (the split fp16 path needs aligned rows); both meet the oracle."""
    say("vptq unaligned codebook")
    W, U, C = make_case(9, 48, 70, 8, 300)
    buf = torch.empty(C.size + 1, dtype=torch.float32, device="cuda")
    Cu = buf[1:].view(C.shape)
    Cu.copy_(torch.from_numpy(C))
    assert Cu.data_ptr() % 16 != 0
    idx, What, E = vq.vptq(dev(W), dev(U), 8, Cu, 16, want_E=True)
    compare(W, U, C, 8, 16, host(idx).reshape(70, 6), host(What), host(E))


@pytest.mark.parametrize("wscale", [1e-6, 1e4])
def test_vptq_scale_extremes(wscale):
    """Working values far below or far above the codebook's scale: the
    per-wavefront power-of-two scale is clamped (tiny columns) or the norm
    term's factor shrinks (huge columns, where the decisions sit at relative
    distance margins near 1e-7 and most go to the exact search); the oracle
    is met bit for bit either way."""
    say("vptq scale", wscale)
    W, U, C = make_case(10, 64, 40, 8, 200)
    idx, What, E = vq.vptq(dev(W * np.float32(wscale)), dev(U), 8, dev(C), 8, want_E=True)
    compare(W * np.float32(wscale), U, C, 8, 8, host(idx).reshape(40, 8), host(What), host(E))


def test_vptq_zero_codebook():
    """Every centroid zero: all distances tie and index 0 wins everywhere."""
    say("vptq zero codebook")
    W, U, _ = make_case(11, 32, 24, 8, 4)
    C = np.zeros((600, 8), np.float32)
    idx, What, E = vq.vptq(dev(W), dev(U), 8, dev(C), 8, want_E=True)
    assert not host(idx).any()
    assert not host(What).any()
    compare(W, U, C, 8, 8, host(idx).reshape(24, 4), host(What), host(E))


def test_vptq_fullsize_sampled_rows():
    """4096 x 11008 with K = 65536, V = 8, B = 128, H = X^T X of the workload's
    activations, GPTQ's U; 32 row groups (256 rows) against the oracle run on
    those rows (groups of V rows evolve independently given U and C)."""
    cfg = configs.get(4)
    M, N, V, K, B = cfg.M, cfg.N, 8, cfg.K1, 128
    say("vptq full size: hessian")
    W = synth.make_weight(cfg.cid, M, N, cfg.scale, cfg.nu, cfg.bf16)
    H = synth.make_hessian(cfg.cid, N, cfg.T, cfg.n_ch, cfg.ch_gain)
    U = oracle.inverse_hessian_factor(H).astype(np.float32)
    del H
    g = np.random.default_rng([cfg.cid, 97])
    cols = W.T.reshape(-1, V)
    C = cols[np.sort(g.choice(cols.shape[0], K, replace=False))].copy()
    say("vptq full size: GPU")
    idx, What, E = vq.vptq(dev(W), dev(U), V, dev(C), B, want_E=True)
    idx, What, E = host(idx).reshape(N, M // V), host(What), host(E)
    groups = np.sort(g.choice(M // V, 32, replace=False))
    rows = np.concatenate([np.arange(q * V, q * V + V) for q in groups])
    say("vptq full size: oracle on groups", groups)
    compare(W, U, C, V, B, idx[:, groups], What[rows], E[rows], rows=rows)


@pytest.mark.parametrize("N,T,damp", [(1, 4, 0.01), (5, 3, 0.01), (33, 40, 0.01), (64, 20, 0.1), (100, 300, 0.01),
                                      (129, 200, 0.01), (300, 64, 0.01), (517, 300, 0.01)])
def test_hessian_factor_matches_oracle(N, T, damp):
    """U from the float64 Cholesky route against numpy's inverse-then-Cholesky
    (float64), both stored float32: |dU| <= 1e-5 max|U|; strict lower triangle 0.
    T < N cases make X^T X singular, so the damping carries them.  N = 129,
    300 and 517 cross the 128-column panels (a one-column last panel, ragged
    sub-panels)."""
    say("hessian factor N =", N)
    g = np.random.default_rng([71, N])
    X = g.standard_normal((T, N))
    X[:, g.choice(N, max(1, N // 10), replace=False)] *= 10.0
    H = (X.T @ X).astype(np.float32)
    ref = oracle.inverse_hessian_factor(H.astype(np.float64), damp)
    got = host(vq.hessian_factor(dev(H), damp))
    assert np.all(np.tril(got, -1) == 0.0)
    err = np.abs(got.astype(np.float64) - ref)
    assert err.max() <= 1e-5 * np.abs(ref).max(), float(err.max() / np.abs(ref).max())


def test_hessian_factor_fullsize():
    """N = 11008 with the 4096 x 11008 workload's activations (T = 1024 < N)."""
    cfg = configs.get(4)
    say("hessian factor full size")
    H = synth.make_hessian(cfg.cid, cfg.N, cfg.T, cfg.n_ch, cfg.ch_gain)
    got = host(vq.hessian_factor(dev(H), 0.01))
    ref = oracle.inverse_hessian_factor(H.astype(np.float64), 0.01)
    err = np.abs(got.astype(np.float64) - ref)
    say("  max |dU| / max |U| = %.3g" % float(err.max() / np.abs(ref).max()))
    assert np.all(np.tril(got, -1) == 0.0)
    assert err.max() <= 1e-5 * np.abs(ref).max()
