"""Parity of every HIP step with the CPU oracle on seeded inputs (GPU).

Bar: indices, CSR arrays, masks, residuals and reconstructions bit-exact;
centroids within 1e-5 of the oracle's per-centroid max norm; objectives
within 1e-5 relative (float64 sums taken in a different order differ only
in the last bits).  Sizes span several MFMA tiles, LDS chunks and sort
blocks, with ragged tails; the edge cases are K = 1, K = n_sub, d < 8,
fully masked sub-vectors, exact ties, nnz = 0 and nnz = M*N.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (bits_equal, centroid_close, dev, host, index_flips_allowed, keep_from_mask,
                      mask_from_keep)
from hessian_weighted_vector_amd import synth
from hessian_weighted_vector_amd import vq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(seed, M, N, d, K, masked=True, with_rho=True, p=0.03):
    g = np.random.default_rng([99, seed])
    inp = synth.small_case(seed, M, N, d=d)
    W, h = inp["W"], inp["h"]
    n_sub = M * N // d
    C, taken = oracle.init(W, d, inp["perm1"], K)
    assert taken == K
    C = C + (0.002 * g.standard_normal(C.shape)).astype(np.float32)
    keep = None
    if masked:
        nz = oracle.nnz(M, N, p)
        _, _, _, keep = oracle.select(W, h, nz)
        keep = keep.copy()
        if n_sub > 3:
            keep.reshape(-1, d)[n_sub // 3] = 0          # one fully masked sub-vector
    rho = g.uniform(0.5, 2.0, M).astype(np.float32) if with_rho else None
    return W, h, C, keep, rho


ASSIGN_CASES = [
    # (seed, M, N, d, K, masked, rho)
    (1, 64, 64, 8, 16, True, True),
    (2, 37, 40, 8, 33, True, False),       # ragged: n_sub = 185, K not a multiple of 32
    (3, 128, 256, 8, 256, True, True),
    (4, 256, 512, 8, 1000, True, True),    # several LDS chunks, partial last chunk
    (5, 16, 24, 3, 7, True, True),         # d = 3
    (6, 8, 8, 1, 5, False, False),         # d = 1
    (7, 200, 64, 4, 100, True, False),
    (8, 1, 8, 8, 1, False, False),         # one sub-vector, K = 1
    (9, 50, 80, 8, 500, False, True),      # K = n_sub
    (10, 96, 96, 6, 200, True, True),
    (11, 256, 512, 8, 3000, True, True),   # long codebook: per-tile tracking, last tile re-formed
    (12, 300, 96, 3, 2500, True, False),   # long codebook, d = 3, ragged last chunk
    (13, 3, 6400, 8, 2200, True, True),    # long codebook, masked, fewer than 4 rows (no block classes)
    (14, 1040, 8096, 8, 3, True, True),    # one-chunk search: > 4096 groups of 256, workgroups take two
]


@pytest.mark.parametrize("case", ASSIGN_CASES, ids=[str(c[:5]) for c in ASSIGN_CASES])
def test_assign_matches_oracle_bitwise(case):
    seed, M, N, d, K, masked, with_rho = case
    say("assign case", case)
    W, h, C, keep, rho = _case(seed, M, N, d, K, masked, with_rho)
    ref_idx, ref_dist = oracle.assign(W, h, rho, keep, d, C)
    ws = vq.workspace(M, N, d, K)
    mask = None if keep is None else dev(mask_from_keep(keep, d))
    idx, dist = vq.assign(dev(W), dev(h), None if rho is None else dev(rho), mask, d, dev(C), ws,
                          want_dist=True)
    gi = host(idx)
    assert bits_equal(gi, ref_idx), np.flatnonzero(gi != ref_idx)[:10]
    assert bits_equal(host(dist), ref_dist.astype(np.float32))


def _many_pattern_keep(M, N, d, seed):
    """Per column block, mask bytes drawn from six candidates (0xFF, fully
    masked, among them) with uneven frequencies, so most blocks have more than
    four classes; block 0 has five bytes with equal counts (the four lowest
    bytes are its classes) and block 1 a single byte."""
    g = np.random.default_rng([77, seed])
    nb = N // d
    mb = np.zeros((M, nb), np.uint8)
    for b in range(nb):
        cand = g.choice(256, 6, replace=False).astype(np.uint8)
        cand[g.integers(6)] = 0xFF
        mb[:, b] = cand[g.choice(6, M, p=g.dirichlet(np.ones(6)))]
    assert M % 5 == 0
    mb[:, 0] = np.repeat(np.array([9, 200, 3, 0xFF, 17], np.uint8), M // 5)[g.permutation(M)]
    mb[:, 1] = 0x24
    return keep_from_mask(mb.ravel(), M, N, d)


@pytest.mark.parametrize("mode", ["no-mask", "zero-mask", "salient", "many-patterns"])
def test_assign_long_codebook_block_shared_weights(mode):
    # K > 2048: sub-vectors whose mask byte is one of their column block's
    # four most frequent take the two-MFMA form, the others (their own mask
    # byte) the three-MFMA form
    say("assign long codebook", mode)
    M, N, d, K = 640, 256, 8, 2600          # 2.5 row groups of 256, ragged codebook chunk
    W, h, C, keep, rho = _case(41, M, N, d, K, masked=(mode != "no-mask"), with_rho=True)
    if mode == "zero-mask":
        keep = np.ones_like(keep)
    if mode == "many-patterns":
        keep = _many_pattern_keep(M, N, d, 41)
    ref_idx, ref_dist = oracle.assign(W, h, rho, keep, d, C)
    ws = vq.workspace(M, N, d, K)
    mask = None if keep is None else dev(mask_from_keep(keep, d))
    idx, dist = vq.assign(dev(W), dev(h), dev(rho), mask, d, dev(C), ws, want_dist=True)
    assert bits_equal(host(idx), ref_idx), np.flatnonzero(host(idx) != ref_idx)[:10]
    assert bits_equal(host(dist), ref_dist.astype(np.float32))


def test_assign_far_outlier_goes_to_exact_search():
    # a sub-vector ~1e15 times larger than every centroid: its scaled weights
    # cannot share the codebook's scale, so the search leaves it to the exact path
    say("assign far outlier")
    M, N, d, K = 256, 128, 8, 2100
    W, h, C, keep, rho = _case(43, M, N, d, K, masked=False, with_rho=False)
    W = W.copy()
    W[5, 8:16] = np.float32(3e13) * np.arange(1, 9, dtype=np.float32)
    W[77, 0:8] = -np.float32(1e14)
    ref_idx, ref_dist = oracle.assign(W, h, None, None, d, C)
    ws = vq.workspace(M, N, d, K)
    idx, dist = vq.assign(dev(W), dev(h), None, None, d, dev(C), ws, want_dist=True)
    assert bits_equal(host(idx), ref_idx), np.flatnonzero(host(idx) != ref_idx)[:10]
    assert bits_equal(host(dist), ref_dist.astype(np.float32))
    assert vq.assign_exact_count(ws, M * N // d, K) >= 2


def test_assign_exact_ties_go_to_lowest_index():
    say("assign ties")
    g = np.random.default_rng(5)
    M, N, d, K = 32, 64, 8, 70
    W = g.standard_normal((M, N)).astype(np.float32)
    h = np.ones(N, np.float32)
    C = W.reshape(-1, d)[:K].copy()
    C[40] = C[3]                # duplicate centroid: never chosen over 3
    C[69] = C[10]
    ref, _ = oracle.assign(W, h, None, None, d, C)
    ws = vq.workspace(M, N, d, K)
    idx = host(vq.assign(dev(W), dev(h), None, None, d, dev(C), ws))
    assert bits_equal(idx, ref)
    assert not np.any(idx == 40) and not np.any(idx == 69)
    assert vq.assign_exact_count(ws, M * N // d, K) > 0   # exact ties cannot be certified


@pytest.mark.parametrize("case", ["some-ties", "all-ties"])
def test_assign_long_codebook_ties_go_to_lowest_index(case):
    # a codebook longer than 2048 with duplicated rows, and sub-vectors equal
    # to codebook rows: exact ties cannot be certified, so the re-search takes
    # them (the chunk-minimum path for up to 32768 of them, the full scan for
    # the rest when "all-ties" floods the list with 65536)
    say("assign long-codebook ties", case)
    g = np.random.default_rng([7, len(case)])
    M, N, d, K = 512, 1024, 8, 4096
    n_sub = M * N // d
    C = g.standard_normal((K, d)).astype(np.float32)
    if case == "some-ties":
        C[2900] = C[5]
        C[1500] = C[700]
        C[4095] = C[0]
        rows = g.integers(0, K, size=n_sub)
        rows[: n_sub // 4] = g.choice([5, 700, 0, 2900, 1500, 4095], size=n_sub // 4)
    else:
        C[1::2] = C[0::2]                       # every centroid twice
        rows = g.integers(0, K, size=n_sub)
    X = C[rows].reshape(M, N)
    h = (0.5 + g.random(N)).astype(np.float32)
    ref, ref_d = oracle.assign(X, h, None, None, d, C)
    ws = vq.workspace(M, N, d, K)
    idx, dist = vq.assign(dev(X), dev(h), None, None, d, dev(C), ws, want_dist=True)
    assert bits_equal(host(idx), ref), np.flatnonzero(host(idx) != ref)[:10]
    assert bits_equal(host(dist), ref_d.astype(np.float32))
    got = host(idx)
    if case == "some-ties":
        assert not np.any(np.isin(got, [2900, 1500, 4095]))
    else:
        assert not np.any(got % 2 == 1)
        assert vq.assign_exact_count(ws, n_sub, K) > 32768


def test_assign_deterministic_and_mostly_certified():
    say("assign determinism")
    W, h, C, keep, rho = _case(21, 256, 512, 8, 512)
    M, N = W.shape
    ws = vq.workspace(M, N, 8, 512)
    args = (dev(W), dev(h), dev(rho), dev(mask_from_keep(keep, 8)), 8, dev(C), ws)
    a = host(vq.assign(*args))
    n_exact = vq.assign_exact_count(ws, M * N // 8, 512)
    b = host(vq.assign(*args))
    assert bits_equal(a, b)
    assert n_exact < 0.05 * (M * N // 8), n_exact


UPDATE_CASES = [(1, 64, 64, 8, 16), (2, 37, 40, 8, 33), (3, 256, 512, 8, 300), (4, 300, 512, 8, 4000),
                (5, 16, 24, 3, 7), (6, 64, 256, 8, 256), (7, 512, 512, 8, 2048)]


@pytest.mark.parametrize("case", UPDATE_CASES, ids=[str(c) for c in UPDATE_CASES])
def test_update_matches_oracle(case):
    seed, M, N, d, K = case
    say("update case", case)
    W, h, C, keep, rho = _case(seed, M, N, d, K)
    idx, _ = oracle.assign(W, h, rho, keep, d, C)
    idx[: min(5, idx.size)] = K - 1         # make sure the last centroid has members
    Cref, cref, Jref = oracle.update(W, h, rho, keep, d, idx, C)
    ws = vq.workspace(M, N, d, K)
    Cg = dev(C)
    counts, J = vq.update(dev(W), dev(h), dev(rho), dev(mask_from_keep(keep, d)), d, dev(idx), Cg, ws)
    ok, bad = centroid_close(host(Cg), Cref)
    assert ok, bad[:10]
    assert np.array_equal(host(counts), cref)
    assert abs(float(host(J)[0]) - Jref) <= 1e-12 * abs(Jref)
    # empty centroids keep their value bit for bit
    empty = cref == 0
    assert bits_equal(host(Cg)[empty], C[empty])
    # with at most 32768 members per 256-centroid group every sum is taken in
    # ascending sub-vector order, as in the oracle: the centroids agree bit for bit
    if np.bincount(idx.astype(np.int64) >> 8).max() <= 32768:
        assert bits_equal(host(Cg), Cref)


@pytest.mark.parametrize("case", [(8, 1024, 1024, 8, 200, 0.0), (9, 1024, 768, 8, 700, 0.6),
                                  (10, 700, 1024, 8, 5000, 0.45)],
                         ids=["one-group-4-pieces", "skewed-700", "skewed-5000"])
def test_update_many_members_per_group(case):
    # groups of 256 centroids with more members than one LDS piece holds: the
    # pieces' partial sums are combined in a second pass
    seed, M, N, d, K, skew = case
    say("update multi-piece", case)
    W, h, C, keep, rho = _case(seed, M, N, d, K)
    g = np.random.default_rng([99, seed, 1])
    idx, _ = oracle.assign(W, h, rho, keep, d, C)
    hot = g.random(idx.size) < skew
    idx[hot] = g.integers(0, min(K, 256), size=int(hot.sum()))   # crowd the first group
    idx[: min(5, idx.size)] = K - 1
    Cref, cref, Jref = oracle.update(W, h, rho, keep, d, idx, C)
    ws = vq.workspace(M, N, d, K)
    Cg = dev(C)
    counts, J = vq.update(dev(W), dev(h), dev(rho), dev(mask_from_keep(keep, d)), d, dev(idx), Cg, ws)
    ok, bad = centroid_close(host(Cg), Cref)
    assert ok, bad[:10]
    assert np.array_equal(host(counts), cref)
    assert abs(float(host(J)[0]) - Jref) <= 1e-12 * abs(Jref)


@pytest.mark.parametrize("case", [(11, 256, 512, 8, 1000), (12, 200, 96, 3, 1500), (13, 90, 70, 7, 400)],
                         ids=["empty-group-d8", "empty-group-d3", "empty-group-d7"])
def test_update_empty_centroid_group(case):
    # K > 256 with no member in centroids [128, 256): their counts are zero and
    # their rows of C stay as they were, bit for bit; d < 8 takes the scalar paths
    seed, M, N, d, K = case
    say("update empty group", case)
    W, h, C, keep, rho = _case(seed, M, N, d, K)
    g = np.random.default_rng([99, seed, 2])
    idx, _ = oracle.assign(W, h, rho, keep, d, C)
    hole = (idx >= 128) & (idx < 256)
    idx[hole] = g.integers(0, 128, size=int(hole.sum()))
    idx[: min(5, idx.size)] = K - 1
    Cref, cref, Jref = oracle.update(W, h, rho, keep, d, idx, C)
    assert (cref[128:256] == 0).all()
    ws = vq.workspace(M, N, d, K)
    Cg = dev(C)
    counts, J = vq.update(dev(W), dev(h), dev(rho), dev(mask_from_keep(keep, d)), d, dev(idx), Cg, ws)
    assert np.array_equal(host(counts), cref)
    assert bits_equal(host(Cg), Cref)
    assert abs(float(host(J)[0]) - Jref) <= 1e-12 * abs(Jref)


@pytest.mark.parametrize("K", [256, 3000], ids=["one-bucket", "buckets"])
def test_update_sorted_indices(K):
    # indices sorted by centroid: every sub-chunk of the reduction belongs to
    # one or two centroids, so single lanes walk a thousand members in a row
    seed, M, N, d = 41, 512, 1024, 8
    say("update sorted indices", K)
    W, h, C, keep, rho = _case(seed, M, N, d, K)
    n_sub = M * N // d
    g = np.random.default_rng([99, seed, 3])
    idx = np.sort(g.integers(0, K, size=n_sub)).astype(np.uint16)
    Cref, cref, Jref = oracle.update(W, h, rho, keep, d, idx, C)
    ws = vq.workspace(M, N, d, K)
    Cg = dev(C)
    counts, J = vq.update(dev(W), dev(h), dev(rho), dev(mask_from_keep(keep, d)), d, dev(idx), Cg, ws)
    ok, bad = centroid_close(host(Cg), Cref)
    assert ok, bad[:10]
    assert np.array_equal(host(counts), cref)
    assert abs(float(host(J)[0]) - Jref) <= 1e-12 * abs(Jref)


def test_update_deterministic():
    say("update determinism")
    W, h, C, keep, rho = _case(31, 512, 1024, 8, 4096)
    M, N = W.shape
    idx, _ = oracle.assign(W, h, rho, keep, 8, C)
    ws = vq.workspace(M, N, 8, 4096)
    outs = []
    for _ in range(2):
        Cg = dev(C)
        vq.update(dev(W), dev(h), dev(rho), dev(mask_from_keep(keep, 8)), 8, dev(idx), Cg, ws)
        outs.append(host(Cg))
    assert bits_equal(outs[0], outs[1])


SELECT_CASES = [(1, 64, 64, 8, 0.03), (2, 37, 40, 8, 0.3), (3, 300, 520, 8, 0.01), (4, 16, 24, 3, 0.0),
                (5, 16, 24, 8, 1.0), (6, 1, 4096, 8, 0.05), (7, 2000, 64, 4, 0.02)]


@pytest.mark.parametrize("case", SELECT_CASES, ids=[str(c) for c in SELECT_CASES])
def test_select_matches_oracle_bitwise(case):
    seed, M, N, d, p = case
    say("select case", case)
    inp = synth.small_case(seed, M, N, d=d)
    W, h = inp["W"], inp["h"]
    if seed == 3:
        W = synth.round_bf16(W * 8)            # many repeated values -> exact ties at the threshold
    nz = oracle.nnz(M, N, p)
    rp, col, val, keep = oracle.select(W, h, nz)
    ws = vq.workspace(M, N, d, 1)
    grp, gcol, gval, gmask = vq.sparse_select(dev(W), dev(h), d, nz, ws)
    assert bits_equal(host(grp), rp)
    assert bits_equal(host(gcol), col)
    assert bits_equal(host(gval), val)
    assert bits_equal(host(gmask), mask_from_keep(keep, d))


def test_binorm_matches_oracle():
    say("binorm")
    inp = synth.small_case(41, 300, 520, d=8)
    W, h = synth.round_bf16(inp["W"]), inp["h"]
    W[7] = 0.0
    Wp, r, c, hcol, rho = oracle.binorm(W, h)
    ws = vq.workspace(300, 520, 8, 1)
    gWp, gr, gc, ghcol, grho = [host(t) for t in vq.binorm(dev(W), dev(h), ws)]
    # float64 sums in another order: equal bits except in rare rounding ties
    for a, b in [(gr, r), (gc, c), (ghcol, hcol), (grho, rho), (gWp, Wp)]:
        ulp = np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))
        assert ulp.max() <= 1
        assert (ulp > 0).mean() < 1e-3


def test_init_matches_oracle_bitwise():
    say("init")
    inp = synth.small_case(51, 64, 128, d=8)
    W = synth.round_bf16(inp["W"] * 0.01)      # coarse values: many repeated sub-vectors? few
    W.reshape(-1, 8)[::3] = W.reshape(-1, 8)[0]  # force repeats
    for K in (1, 50, 600):
        Cref, taken = oracle.init(W, 8, inp["perm1"], K)
        ws = vq.workspace(64, 128, 8, K)
        if taken < K:
            with pytest.raises(vq.VQError) as e:
                vq.init(dev(W), 8, inp["perm1"], K, ws)
            assert e.value.status == vq.VQ_ERR_INIT
        else:
            assert bits_equal(host(vq.init(dev(W), 8, inp["perm1"], K, ws)), Cref)


def test_init_walk_beyond_first_chunk_matches_oracle():
    """The device dedupes the first chunk of the walk (65536 positions here); when
    that chunk holds fewer than K distinct rows the walk is done again on the host
    and continues into the next chunk.  Both paths against the oracle, bitwise."""
    say("init beyond the first chunk")
    g = np.random.default_rng([52, 0])
    M, N, d = 1024, 1024, 8
    W = (0.02 * g.standard_normal((M, N))).astype(np.float32)
    perm = g.permutation(M * N // d).astype(np.int32)
    base = (0.02 * g.standard_normal((500, d))).astype(np.float32)
    W.reshape(-1, d)[perm[:65536]] = base[np.arange(65536) % 500]    # 500 distinct rows in the first chunk
    for K in (400, 1000):
        Cref, taken = oracle.init(W, d, perm, K)
        assert taken == K
        ws = vq.workspace(M, N, d, K)
        assert bits_equal(host(vq.init(dev(W), d, perm, K, ws)), Cref)


def test_residual_and_reconstruct_bitwise():
    say("residual + reconstruct")
    W, h, C, keep, rho = _case(61, 128, 256, 8, 64)
    M, N = W.shape
    idx, _ = oracle.assign(W, h, rho, keep, 8, C)
    R = oracle.residual(W, 8, C, idx)
    gR = host(vq.residual(dev(W), 8, dev(C), dev(idx)))
    assert bits_equal(gR, R)
    C2 = (0.001 * np.random.default_rng(3).standard_normal((16, 8))).astype(np.float32)
    idx2 = np.random.default_rng(4).integers(0, 16, M * N // 8).astype(np.uint16)
    r = np.random.default_rng(5).uniform(0.5, 2, M).astype(np.float32)
    c = np.random.default_rng(6).uniform(0.5, 2, N).astype(np.float32)
    rp, col, val, _ = oracle.select(W, h, 300)
    for args in [(None, None, None, None), (C2, idx2, None, None), (C2, idx2, r, c)]:
        C2a, i2, ra, ca = args
        ref = oracle.reconstruct(M, N, 8, C, idx, C2a, i2, ra, ca, rp, col, val)
        got = vq.reconstruct(M, N, 8, dev(C), dev(idx), None if C2a is None else dev(C2a),
                             None if i2 is None else dev(i2), None if ra is None else dev(ra),
                             None if ca is None else dev(ca), dev(rp), dev(col), dev(val))
        assert bits_equal(host(got), ref)


def _compare_fit(o, g, d, K2, tol_c=1e-5):
    assert bits_equal(host(g["row_ptr"]), o["row_ptr"])
    assert bits_equal(host(g["col"]), o["col"])
    assert bits_equal(host(g["val"]), o["val"])
    M, N = o["keep"].shape
    assert bits_equal(host(g["mask"]), mask_from_keep(o["keep"], d))
    assert bits_equal(host(g["idx1"]), o["idx1"])
    ok, bad = centroid_close(host(g["C1"]), o["C1"], tol_c)
    assert ok, bad[:10]
    if K2:
        assert bits_equal(host(g["idx2"]), o["idx2"])
        ok, bad = centroid_close(host(g["C2"]), o["C2"], tol_c)
        assert ok, bad[:10]
    assert np.allclose(g["J"], o["J"], rtol=1e-5, atol=0)
    # the reconstruction is bitwise when the trajectories agree bitwise
    return bits_equal(host(g["W_hat"]), o["What"])


@pytest.mark.parametrize("binorm", [False, True])
def test_fit_tiny_config_matches_oracle(binorm):
    from hessian_weighted_vector_amd import configs
    cfg = configs.get(1)
    say("fit config", cfg.name, "binorm", binorm)
    inp = synth.make_inputs(cfg)
    K2, T2 = (32, 4) if binorm else (cfg.K2, cfg.T2)
    o = oracle.fit(inp["W"], inp["h"], cfg.d, cfg.K1, cfg.T1, K2, T2, cfg.p, binorm, True,
                   inp["perm1"], inp["perm2"])
    g = vq.fit(dev(inp["W"]), dev(inp["h"]), cfg.d, cfg.K1, cfg.T1, K2, T2, cfg.p, binorm, True,
               inp["perm1"], inp["perm2"])
    same = _compare_fit(o, g, cfg.d, K2)
    assert same
    J = g["J"]
    assert np.all(J[1:cfg.T1 + 1] <= J[:cfg.T1] * (1 + 1e-6))
    assert g["bpw"] == pytest.approx(oracle.bits_per_weight(cfg.M, cfg.N, cfg.d, cfg.K1, K2, o["nnz"], 32, binorm))


def test_fit_unmasked_and_degenerate():
    say("fit degenerate")
    inp = synth.small_case(71, 16, 32, d=8)
    W, h = inp["W"], inp["h"]
    n_sub = 64
    # K = n_sub and p = 0: exact reconstruction, J = 0
    g = vq.fit(dev(W), dev(h), 8, n_sub, 3, 0, 0, 0.0, perm1=inp["perm1"])
    assert np.all(g["J"] == 0) and bits_equal(host(g["W_hat"]), W)
    # p = 1: every weight held exactly
    g = vq.fit(dev(W), dev(h), 8, 4, 2, 2, 2, 1.0, perm1=inp["perm1"], perm2=inp["perm2"])
    assert np.all(g["J"] == 0) and bits_equal(host(g["W_hat"]), W)
    # mask_outliers = 0 (salient weights stay in the clustering, still overwritten)
    o = oracle.fit(W, h, 8, 12, 3, 5, 2, 0.05, False, False, inp["perm1"], inp["perm2"])
    g = vq.fit(dev(W), dev(h), 8, 12, 3, 5, 2, 0.05, False, False, inp["perm1"], inp["perm2"])
    assert _compare_fit(o, g, 8, 5)


def _replay_stage(X, hc, rh, keep, d, C, T):
    """The oracle's Lloyd stage step by step: (codebook, indices, centroids left
    without members after each update)."""
    empty = []
    for _ in range(T):
        idx, _ = oracle.assign(X, hc, rh, keep, d, C)
        C, counts, _ = oracle.update(X, hc, rh, keep, d, idx, C)
        empty.append(int(np.count_nonzero(counts == 0)))
    idx, _ = oracle.assign(X, hc, rh, keep, d, C)
    return C, idx, empty


@pytest.mark.parametrize("case", ["ties", "binorm"])
def test_fit_empty_centroid_history_matches_oracle(case):
    # "ties": weights on three levels and zero column weights on the last four
    # dimensions of every block, so distinct seeds coincide under the weighted
    # distance; the lowest index takes every tie and the others stay empty (and
    # keep their value) at every update.  "binorm": a plain random case (no
    # centroid goes empty), compared the same way.
    say("fit empty history", case)
    inp = synth.small_case(83, 64, 128, d=8)
    W, h = inp["W"], inp["h"]
    binorm = case == "binorm"
    if case == "ties":
        g = np.random.default_rng([83, 1])
        W = (0.01 * g.integers(0, 3, size=W.shape)).astype(np.float32)
        h = h.copy()
        h[(np.arange(h.size) % 8) >= 4] = 0.0
    d, K1, T1, K2, T2, p = 8, 400, 6, 100, 4, 0.02
    o = oracle.fit(W, h, d, K1, T1, K2, T2, p, binorm, True, inp["perm1"], inp["perm2"])
    X, hc, rh, keep = o["Wp"], o["hcol"], (o["rho"] if binorm else None), o["keep"]
    C1, taken = oracle.init(X, d, inp["perm1"], K1)
    assert taken == K1
    C1, idx1, e1 = _replay_stage(X, hc, rh, keep, d, C1, T1)
    assert bits_equal(C1, o["C1"]) and np.array_equal(idx1, o["idx1"])      # the replay is the fit
    R = oracle.residual(X, d, C1, idx1)
    C2, taken = oracle.init(R, d, inp["perm2"], K2)
    assert taken == K2
    C2, idx2, e2 = _replay_stage(R, hc, rh, keep, d, C2, T2)
    assert bits_equal(C2, o["C2"]) and np.array_equal(idx2, o["idx2"])
    expect = np.array(e1 + e2, np.int64)
    if case == "ties":
        assert expect.min() > 0                                             # the case exercises empties
    g = vq.fit(dev(W), dev(h), d, K1, T1, K2, T2, p, binorm, True, inp["perm1"], inp["perm2"])
    assert np.array_equal(host(g["idx1"]), o["idx1"]) and np.array_equal(host(g["idx2"]), o["idx2"])
    assert np.array_equal(g["empty"], expect), (g["empty"], expect)


def test_fit_smollm2_config_matches_oracle():
    """The 2048 x 2048 workload end to end (oracle: tens of seconds)."""
    from hessian_weighted_vector_amd import configs
    cfg = configs.get(2)
    say("fit config", cfg.name)
    inp = synth.make_inputs(cfg)
    o = oracle.fit(inp["W"], inp["h"], cfg.d, cfg.K1, cfg.T1, cfg.K2, cfg.T2, cfg.p, cfg.binorm, True,
                   inp["perm1"], inp["perm2"])
    say("oracle done")
    g = vq.fit(dev(inp["W"]), dev(inp["h"]), cfg.d, cfg.K1, cfg.T1, cfg.K2, cfg.T2, cfg.p, cfg.binorm, True,
               inp["perm1"], inp["perm2"])
    same = _compare_fit(o, g, cfg.d, cfg.K2)
    assert same
