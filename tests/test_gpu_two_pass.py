"""The two-pass search of long codebooks against the oracle (GPU).

With a workspace that has room for it, a long codebook (more than 2048
centroids) is searched in two passes: a coarse pass (one fp16 MFMA per tile)
names each sub-vector's candidate groups of 1024 centroids, the candidates are
searched in the general form and the winners certified.  A sub-vector with
more than three candidate groups is searched over the whole codebook.  With a
workspace of exactly the required size the one-pass search runs instead.
Both must give the oracle's indices and distances bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
from gpu_util import bits_equal, dev, host, mask_from_keep
from hessian_weighted_vector_amd import synth
from hessian_weighted_vector_amd import vq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _min_workspace(args, full):
    """Smallest byte count vq_assign accepts for these arguments (the library
    checks the size before it launches anything)."""
    lo, hi = 0, full.numel()          # lo refused, hi accepted
    while hi - lo > 1:
        mid = (lo + hi) // 2
        try:
            vq.assign(*args, full[:mid])
            hi = mid
        except vq.VQError as e:
            assert e.status == vq.VQ_ERR_WORKSPACE, e
            lo = mid
    return hi


def _salient_case(seed, M, N, d, K):
    g = np.random.default_rng([123, seed])
    inp = synth.small_case(seed, M, N, d=d)
    W, h = inp["W"], inp["h"]
    C, taken = oracle.init(W, d, inp["perm1"], K)
    assert taken == K
    C = C + (0.002 * g.standard_normal(C.shape)).astype(np.float32)
    _, _, _, keep = oracle.select(W, h, oracle.nnz(M, N, 0.02))
    rho = g.uniform(0.5, 2.0, M).astype(np.float32)
    return W, h, C, keep.copy(), rho


@pytest.mark.parametrize("masked", [True, False], ids=["salient", "no-mask"])
def test_one_pass_and_two_pass_match_oracle(masked):
    say("one-pass vs two-pass", masked)
    M, N, d, K = 512, 1024, 8, 4500            # five groups of 1024, the last one ragged
    W, h, C, keep, rho = _salient_case(3, M, N, d, K)
    if not masked:
        keep = None
    ref_idx, ref_dist = oracle.assign(W, h, rho, keep, d, C)
    mask = None if keep is None else dev(mask_from_keep(keep, d))
    full = vq.workspace(M, N, d, K)
    args = (dev(W), dev(h), dev(rho), mask, d, dev(C))
    i2, d2 = vq.assign(*args, full, want_dist=True)
    assert bits_equal(host(i2), ref_idx), np.flatnonzero(host(i2) != ref_idx)[:10]
    assert bits_equal(host(d2), ref_dist.astype(np.float32))
    n_min = _min_workspace(args, full)
    assert n_min < full.numel()
    i1, d1 = vq.assign(*args, full[:n_min], want_dist=True)
    assert bits_equal(host(i1), ref_idx), np.flatnonzero(host(i1) != ref_idx)[:10]
    assert bits_equal(host(d1), ref_dist.astype(np.float32))


@pytest.mark.parametrize("masked", [False, True], ids=["shared", "own-weights"])
@pytest.mark.parametrize("copies,jitter", [(2, 1e-3), (3, 1e-3), (4, 1e-3), (6, 1e-3), (5, 0.0), (4, 1e-6)],
                         ids=["2-groups", "3-groups", "4-groups", "6-groups", "5-exact-ties", "4-near-ties"])
def test_near_copies_across_groups(copies, jitter, masked):
    # Every sub-vector sits next to a centroid that has near copies in other
    # groups of 1024, so the coarse pass names several candidate groups: up to
    # three are searched as candidates, more send the sub-vector to the
    # whole-codebook search; exact copies are ties that only the exact
    # re-search can settle (lowest index).  "own-weights" masks about a third
    # of the elements at random, so most column blocks have far more than four
    # mask bytes and most sub-vectors are searched with their own weights over
    # the whole codebook (the general form) beside the two-pass search.
    say("near copies", copies, jitter, masked)
    g = np.random.default_rng([31, copies, int(jitter * 1e6)])
    M, N, d, K = 256, 512, 8, 8192
    n_sub = M * N // d
    C = g.standard_normal((K, d)).astype(np.float32)
    base = g.choice(1024, 64, replace=False)
    for c in range(1, copies):
        C[base + 1024 * c] = (C[base] * (1.0 + jitter * g.standard_normal((64, d)))).astype(np.float32)
    rows = g.choice(base, n_sub)
    X = (C[rows] + 0.05 * g.standard_normal((n_sub, d))).astype(np.float32).reshape(M, N)
    h = (0.5 + g.random(N)).astype(np.float32)
    keep = (g.random((M, N)) > 0.3).astype(np.uint8) if masked else None
    if masked:
        keep[:, :d] = 0                          # a fully masked block: index 0 (shared form)
        keep.reshape(-1, d)[g.choice(n_sub, 50, replace=False)] = 0   # and single ones (general form)
    ref, ref_d = oracle.assign(X, h, None, keep, d, C)
    ws = vq.workspace(M, N, d, K)
    mask = dev(mask_from_keep(keep, d)) if masked else None
    idx, dist = vq.assign(dev(X), dev(h), None, mask, d, dev(C), ws, want_dist=True)
    assert bits_equal(host(idx), ref), np.flatnonzero(host(idx) != ref)[:10]
    assert bits_equal(host(dist), ref_d.astype(np.float32))
