"""Randomized fused products and grouped fits against the oracle (GPU).

Fused product: 32 seeded draws of (M, N, d, K1, K2, B), with or without scales
and salient entries, aligned or not, each output held to the bound the
header states (the same check as the fixed cases).  Grouped fit: 24 seeded
draws of the column layout (outlier columns, v0, k0, group count) on top of a
random plain-fit setting, compared with the oracle's grouped fit at the plain
fit's bar (column order, masks, CSR, indices and the reconstruction bit for
bit; codebooks within 1e-5 of each centroid's max norm; objectives within
1e-5 relative).  Draws whose layout does not split the columns must be
refused by the library.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from test_gpu_grouped import compare, perms
from test_gpu_qgemv import check, make_case, run_gpu
from gpu_util import dev
from hessian_weighted_vector_amd import synth, vq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("seed", range(32))
def test_random_qgemv_matches_oracle(seed):
    g = np.random.default_rng([777, seed])
    d = int(g.choice([8, 8, 8, 4, 2, 1, 3, 5, 6, 7]))
    M = int(g.integers(1, 150))
    N = d * int(g.integers(1, 300))
    n_sub = M * N // d
    K1 = int(g.integers(1, min(65536, n_sub) + 1))                 # the library takes K <= n_sub
    K2 = min(int(g.choice([0, int(g.integers(1, 300)), int(g.integers(300, 600))])), n_sub)
    B = int(g.integers(1, 20))
    scales = bool(g.random() < 0.6)
    nnz = None if g.random() < 0.3 else int(g.integers(1, min(12, N) + 1))   # a CSR comes with its arrays
    misalign = bool(g.random() < 0.2)
    say("random qgemv", seed, dict(M=M, N=N, d=d, K1=K1, K2=K2, B=B, scales=scales, nnz=nnz, misalign=misalign))
    cs, X = make_case(900 + seed, M, N, d, K1, K2, B, scales=scales, nnz_per_row=nnz)
    check(cs, X, run_gpu(cs, X, misalign=misalign))


def grouped_draw(seed):
    g = np.random.default_rng([888, seed])
    d = int(g.choice([8, 8, 4, 2]))
    d0 = int(g.choice([4, 2, 1, 8]))
    unit = d * d0 // math.gcd(d, d0)
    M = int(g.integers(4, 64))
    n_out = unit * int(g.integers(0, 4))
    nb_main = int(g.integers(1, 30))
    N = n_out + d * nb_main
    ng = int(g.integers(1, 5))
    w = -(-nb_main // ng)
    smallest = nb_main - (ng - 1) * w               # blocks in the last group (<= 0: no split)
    K1 = K2 = 1
    if smallest > 0:
        K1 = int(g.integers(1, min(M * smallest, 200) + 1))
        K2 = int(g.integers(0, min(M * smallest, 20) + 1)) if g.random() < 0.5 else 0
    K0 = int(g.integers(1, max(2, M * n_out // d0 // 2))) if n_out else 0
    T1, T2, T0 = int(g.integers(0, 4)), int(g.integers(0, 3)), int(g.integers(0, 4))
    p = float(g.choice([0.0, 0.01, 0.03]))
    binorm = bool(g.random() < 0.5)
    return M, N, d, K1, T1, K2, T2 if K2 else 0, p, binorm, n_out, d0, K0, T0, ng, smallest > 0


@pytest.mark.parametrize("seed", range(24))
def test_random_grouped_fit_matches_oracle(seed):
    M, N, d, K1, T1, K2, T2, p, binorm, n_out, d0, K0, T0, ng, splits = grouped_draw(seed)
    say("random grouped", seed, dict(M=M, N=N, d=d, K1=K1, T1=T1, K2=K2, T2=T2, p=p, binorm=binorm, n_out=n_out,
                                     d0=d0, K0=K0, T0=T0, groups=ng, splits=splits))
    prm = vq.grouped_params(M, N, d, K1, T1, K2, T2, p, binorm, True, n_out, d0, K0, T0, ng)
    if not splits:
        # the groups cannot all be non-empty: refused, with no workspace size
        assert vq.grouped_sizes(prm)[0] == 0
        return
    inp = synth.small_case(1200 + seed, M, N, d=d)
    W, h = inp["W"], inp["h"]
    lay = oracle.grouped_layout(N, d, n_out, d0, K0, T0, ng, K1, T1, K2, T2)
    p1, p2 = perms(seed, M, lay)
    try:
        o = oracle.fit_grouped(W, h, d, K1, T1, K2, T2, p, n_out, d0, K0, T0, ng, p1, p2, binorm=binorm)
    except RuntimeError as e:
        assert str(e).endswith(": 1")                 # fewer distinct rows than centroids in some group
        with pytest.raises(vq.VQError) as ge:
            vq.fit_grouped(dev(W), dev(h), prm, p1, p2)
        assert ge.value.status == vq.VQ_ERR_INIT
        return
    gout = vq.fit_grouped(dev(W), dev(h), prm, p1, p2)
    assert compare(o, gout, lay, M, d)
