"""The error bound behind the two-pass search of long codebooks, checked on
the CPU by emulating the coarse pass's arithmetic in float64.

The coarse pass scores a pair with the hi*hi products of the scaled, fp16-split
operands plus the exact class bias.  The search relies on two facts, both
derived in the kernel's comments and checked here on seeded data (heavy-tailed
values, uneven weights with high-energy channels, masked elements, scales from
1e-6 to 1e6):

1. the dropped products are at most a (sqrt(S) + sqrt(D)) in scaled units,
   a = 2^-9 (1 + 2^-10) sqrt(S), with S the sub-vector's weighted energy and D
   the weighted distance (Cauchy-Schwarz and sqrt(B) <= sqrt(S) + sqrt(D));
2. with Ehat the bound written in terms of the coarse score alone, every
   group of centroids whose coarse minimum m satisfies m - Ehat(m) >
   m_1 + Ehat(m_1) holds no centroid at least as near as the exact nearest,
   so the exact argmin (and every tie with it) lies in the candidate groups.

No GPU and no library: this pins the mathematics the kernel is built on.
"""
import numpy as np
import pytest

U = 2.0 ** -24
GROUP = 1024


def f16(a):
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)


def ehat(v, S):
    """Bound on |coarse - exact| from the coarse score v (scaled units)."""
    sqS = np.sqrt(S)
    a = 2.0 ** -9 * (1 + 2.0 ** -10) * sqS
    E0 = 48 * U * (11 * S + 5 * np.abs(v)) + 2
    Dt = np.maximum(v + S, 0.0)
    y = 0.5 * (a + np.sqrt(a * a + 4 * (Dt + a * sqS + E0)))
    return 1.001 * (a * (sqS + y) + E0)


def _case(seed, scale, K=4096, n=300, d=8):
    g = np.random.default_rng([2024, seed])
    C = (scale * g.standard_t(3, size=(K, d))).astype(np.float32).astype(np.float64)
    # sub-vectors near random centroids, some far away
    rows = g.integers(0, K, n)
    X = C[rows] + scale * 0.3 * g.standard_t(4, size=(n, d))
    X[: n // 10] *= 8.0
    X = X.astype(np.float32).astype(np.float64)
    h = g.chisquare(4, size=d)
    h[g.integers(0, d)] *= 400.0                    # a high-energy channel
    W = np.broadcast_to(h, (n, d)).copy()
    W[g.random((n, d)) < 0.05] = 0.0               # masked elements
    W = W.astype(np.float32).astype(np.float64)
    return X, W, C


def _scaled(X, W, C):
    """The coarse pass's operands and exact scores, all in its scaled units."""
    cmax = np.abs(C).max()
    e1 = np.frexp(2 * cmax)[1]
    c_hat = f16(-2 * C * 2.0 ** (15 - e1))                       # [K, d]
    wx = W * X
    mx = np.abs(wx).max(1)
    ex = np.frexp(mx)[1]
    sh = 15 - ex
    x_hat = f16(wx * (2.0 ** sh)[:, None])                         # [n, d]
    shift = sh + (15 - e1)
    scale = 2.0 ** shift
    S = (W * X * X).sum(1) * scale
    B = (C * C) @ W.T                                              # [K, n] exact bias
    exact = (((-2 * C) @ wx.T) + B) * scale[None, :]
    coarse = c_hat @ x_hat.T + B * scale[None, :]
    D = exact + S[None, :]
    return exact, coarse, S, D


@pytest.mark.parametrize("scale", [1e-6, 1e-2, 1.0, 1e3, 1e6])
@pytest.mark.parametrize("seed", [1, 2])
def test_dropped_products_within_bound(seed, scale):
    X, W, C = _case(seed, scale)
    exact, coarse, S, D = _scaled(X, W, C)
    a = 2.0 ** -9 * (1 + 2.0 ** -10) * np.sqrt(S)
    lim = a[None, :] * (np.sqrt(S)[None, :] + np.sqrt(np.maximum(D, 0))) + 2.0
    err = np.abs(coarse - exact)
    assert np.all(err <= lim), float((err / lim).max())
    # the bound is not vacuous: the worst pair uses most of it (0.86-0.92 here)
    assert (err / lim).max() > 0.5


@pytest.mark.parametrize("scale", [1e-3, 1.0, 1e4])
@pytest.mark.parametrize("seed", [3, 4, 5])
def test_exact_argmin_in_candidate_groups(seed, scale):
    X, W, C = _case(seed, scale)
    exact, coarse, S, D = _scaled(X, W, C)
    K, n = exact.shape
    ng = K // GROUP
    gmin = coarse.reshape(ng, GROUP, n).min(1)                     # [ng, n]
    m1 = gmin.min(0)
    Uc = m1 + ehat(m1, S)
    cand = (gmin - ehat(gmin, S[None, :])) <= Uc[None, :]
    best = exact.min(0)
    for s in range(n):
        winners = np.flatnonzero(exact[:, s] == best[s])
        assert np.all(cand[winners // GROUP, s]), s
    # the bound's left side grows with the coarse score
    v = np.linspace(-S.max(), 4 * S.max(), 2001)
    for Ss in S[:20]:
        lv = v - ehat(v, Ss)
        assert np.all(np.diff(lv) > 0)


def test_bound_breaks_without_the_distance_term():
    """A bound that omits a*sqrt(D) is violated on far sub-vectors: the
    distance term is needed, not decoration."""
    X, W, C = _case(7, 1.0)
    exact, coarse, S, D = _scaled(X, W, C)
    a = 2.0 ** -9 * (1 + 2.0 ** -10) * np.sqrt(S)
    lim = a[None, :] * np.sqrt(S)[None, :] + 2.0
    assert np.any(np.abs(coarse - exact) > lim)
