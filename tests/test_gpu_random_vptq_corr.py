"""Randomized Algorithm 1, inverse-Hessian factor and unified correction
against the oracle (GPU).

Algorithm 1: 24 seeded draws of (M, N, V, K, B), V = 1..8 (the scalar and the
vector path), K from 1 to 1500 (one to six 256-centroid chunks), B from 1 to
128 and past N, compared with the oracle's trajectory at the fixed cases' bar
(indices, codebook rows and E identical).

Factor: 12 seeded draws of (N, T, damp), T below N (singular X^T X carried by
the damping) and above, N crossing the 128-column panels; U within 1e-5 of
max |U| of the float64 oracle, its strict lower triangle zero.

Correction: 24 seeded draws of (M, N, d, n_sel, n_res) on tie-heavy inputs,
each running the salient-sub-vector select, the largest-residual select and
the CSR build in sequence on one mask, every result bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
from gpu_util import dev, host, keep_from_mask, mask_from_keep
from hessian_weighted_vector_amd import vq
from test_gpu_correction import tie_case
from test_gpu_vptq import compare, make_case

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def vptq_draw(seed):
    g = np.random.default_rng([5151, seed])
    V = int(g.integers(1, 9))
    M = V * int(g.integers(1, 40))
    N = int(g.integers(1, 220))
    K = int(g.choice([1, int(g.integers(1, 256)), int(g.integers(1, 256)), int(g.integers(256, 1500)),
                      int(g.integers(256, 1500))]))
    B = int(g.choice([1, int(g.integers(1, 129)), int(g.integers(1, 129)), 128]))
    return M, N, V, K, B


@pytest.mark.parametrize("seed", range(24))
def test_random_vptq_matches_oracle(seed):
    M, N, V, K, B = vptq_draw(seed)
    say("random vptq", seed, dict(M=M, N=N, V=V, K=K, B=B))
    W, U, C = make_case(300 + seed, M, N, V, K)
    idx, What, E = vq.vptq(dev(W), dev(U), V, dev(C), B, want_E=True)
    compare(W, U, C, V, B, host(idx).reshape(N, M // V), host(What), host(E))


@pytest.mark.parametrize("seed", range(12))
def test_random_hessian_factor_matches_oracle(seed):
    g = np.random.default_rng([6161, seed])
    N = int(g.choice([int(g.integers(1, 128)), int(g.integers(128, 400))]))
    T = int(g.integers(1, 2 * N + 8))
    damp = float(g.choice([0.01, 0.05, 0.1]))
    say("random factor", seed, dict(N=N, T=T, damp=damp))
    X = g.standard_normal((T, N))
    X[:, g.choice(N, max(1, N // 10), replace=False)] *= 10.0
    H = (X.T @ X).astype(np.float32)
    ref = oracle.inverse_hessian_factor(H.astype(np.float64), damp)
    got = host(vq.hessian_factor(dev(H), damp))
    assert np.all(np.tril(got, -1) == 0.0)
    err = np.abs(got.astype(np.float64) - ref).max()
    assert err <= 1e-5 * np.abs(ref).max(), err / np.abs(ref).max()


def corr_draw(seed):
    g = np.random.default_rng([7171, seed])
    d = int(g.choice([8, 8, 4, 3, 1, 5]))
    M = int(g.integers(1, 200))
    N = d * int(g.integers(1, 80))
    n_sub = M * N // d
    n_sel = int(g.choice([0, int(g.integers(0, n_sub + 1)), int(g.integers(0, n_sub // 4 + 1)), n_sub]))
    n_res = int(g.choice([0, int(g.integers(0, M * N + 1)), int(g.integers(0, M * N // 4 + 1)), 10 ** 7]))
    return M, N, d, n_sel, n_res


@pytest.mark.parametrize("seed", range(24))
def test_random_correction_matches_oracle(seed):
    M, N, d, n_sel, n_res = corr_draw(seed)
    say("random correction", seed, dict(M=M, N=N, d=d, n_sel=n_sel, n_res=n_res))
    W, h, What, keep0, _ = tie_case(500 + seed, M, N)
    k1 = oracle.select_subvectors(W, h, d, n_sel, keep=keep0)
    k2 = oracle.select_residual(W, What, h, n_res, keep=k1)
    rp, col, val = oracle.keep_to_csr(W, k2)
    ws = vq.workspace(M, N, d, 1)
    mask = dev(mask_from_keep(keep0, d))
    dW = dev(W)
    vq.select_subvectors(dW, dev(h), d, n_sel, mask, ws)
    assert np.array_equal(keep_from_mask(host(mask), M, N, d), k1)
    vq.select_residual(dW, dev(What), dev(h), d, n_res, mask, ws)
    assert np.array_equal(keep_from_mask(host(mask), M, N, d), k2)
    n = int(rp[-1])
    grp, gcol, gval = vq.mask_to_csr(dW, mask, d, n, ws)
    assert np.array_equal(host(grp), rp)
    assert np.array_equal(host(gcol)[:n], col)
    assert np.array_equal(host(gval)[:n].view(np.uint32), val.view(np.uint32))
