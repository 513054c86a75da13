"""Pins of the CPU oracle to facts outside itself.

Each pin takes a loaded oracle library and raises AssertionError when the
oracle disagrees with what the pages or the mathematics fix:

  * special cases that reduce to a library routine (scipy's Euclidean vector
    quantizer and k-means, numpy's weighted average and sorts),
  * closed forms and optimality conditions (the weighted mean is the exact
    minimizer of the weighted objective for fixed assignments),
  * invariants (positive rescaling of the Hessian diagonal, RMS of the
    bi-normalized matrix, the objective identity on the reconstruction),
  * degenerate cases (one centroid per sub-vector, every weight salient),
  * brute force on tiny inputs.

The same pins run against deliberately broken copies of the oracle
(test_oracle_mutants.py), which shows that a plausible mistake anywhere in
it fails at least one of them.
"""
import warnings

import numpy as np
import scipy.cluster.vq as scvq
from scipy.spatial.distance import cdist

import oracle as O


def _case(seed, M, N, scale=0.02, nu=4.0, n_ch=2, gain=20.0, T=64):
    g = np.random.default_rng([7, seed])
    W = (scale * g.standard_t(nu, size=(M, N))).astype(np.float32)
    X = g.standard_normal((T, N))
    ch = g.choice(N, min(n_ch, N), replace=False)
    X[:, ch] *= gain
    h = (X * X).sum(0).astype(np.float32)
    return W, h, g


def _scores(W, h):
    # the salience score of the HAS-VQ abstract's decoupling: second-order
    # sensitivity of one weight, h_j * w_ij^2 (fp32: square, then scale)
    return np.float32(h)[None, :] * (W * W)


# --------------------------------------------------------------------------
def pin_select_characterization(lib):
    """Top-nnz by (score desc, linear index asc) is the unique set with:
    exactly nnz members, every member scoring >= every non-member, and at the
    threshold score the members holding the smallest linear indices.  Checked
    on a random case and on all-equal scores (pure index order)."""
    for (M, N, p, seed) in [(40, 24, 0.05, 1), (17, 32, 0.3, 2)]:
        W, h, _ = _case(seed, M, N)
        nz = O.nnz(M, N, p, lib)
        assert nz == int(np.floor(p * M * N))
        rp, col, val, keep = O.select(W, h, nz, lib)
        s = _scores(W, h)
        sel = keep == 0
        assert sel.sum() == nz
        if 0 < nz < M * N:
            tau_in = s[sel].min()
            tau_out = s[~sel].max()
            assert tau_in >= tau_out
            if tau_in == tau_out:
                lin = np.arange(M * N).reshape(M, N)
                assert lin[sel & (s == tau_in)].max() < lin[~sel & (s == tau_in)].min()
        # CSR structure: row pointers, ascending columns, exact values
        assert rp[0] == 0 and rp[-1] == nz and np.all(np.diff(rp) >= 0)
        for i in range(M):
            cs = col[rp[i]:rp[i + 1]]
            assert np.all(np.diff(cs) > 0)
            assert np.all(sel[i, cs])
            assert np.array_equal(val[rp[i]:rp[i + 1]].view(np.uint32), W[i, cs].view(np.uint32))
        assert np.array_equal(np.diff(rp), sel.sum(1))
    # all scores equal: the first nnz linear positions
    M, N = 6, 16
    W = np.full((M, N), 0.5, np.float32)
    h = np.ones(N, np.float32)
    rp, col, val, keep = O.select(W, h, 20, lib)
    assert np.array_equal(np.flatnonzero(keep.ravel() == 0), np.arange(20))


def pin_select_brute_force(lib):
    """Brute force on a tiny case through numpy's lexicographic sort."""
    W, h, _ = _case(11, 12, 16, n_ch=3)
    s = _scores(W, h).ravel()
    order = np.lexsort((np.arange(s.size), -s.astype(np.float64)))
    for nz in [0, 1, 7, 50, 191, 192]:
        _, _, _, keep = O.select(W, h, nz, lib)
        assert set(np.flatnonzero(keep.ravel() == 0)) == set(order[:nz].tolist())


# --------------------------------------------------------------------------
def pin_binorm_invariants(lib):
    """Rows of W / r and columns of W' have unit RMS (fp32 rounding); r c W'
    gives back W; the folded weights keep the original-space objective:
    sum h_j (W - r c V)^2 == sum hcol_j rho_i (W' - V)^2 for any V."""
    W, h, g = _case(3, 24, 40)
    W[5, :] = 0.0  # a zero row takes scale 1
    Wp, r, c, hcol, rho = O.binorm(W, h, lib)
    assert r[5] == 1.0
    Wt = W.astype(np.float64) / r[:, None]
    rows = np.sqrt((Wt ** 2).mean(1))
    assert np.allclose(np.delete(rows, 5), 1.0, rtol=1e-6)
    cols = np.sqrt((Wp.astype(np.float64) ** 2).mean(0))
    assert np.allclose(cols, 1.0, rtol=1e-6)
    back = Wp.astype(np.float64) * c[None, :] * r[:, None]
    assert np.allclose(back, W, rtol=1e-6, atol=0)
    assert np.allclose(hcol, h.astype(np.float64) * c.astype(np.float64) ** 2, rtol=1e-7)
    assert np.allclose(rho, r.astype(np.float64) ** 2, rtol=1e-7)
    V = Wp + 0.1 * g.standard_normal(Wp.shape).astype(np.float32)
    lhs = (h[None, :].astype(np.float64) * (W - r[:, None].astype(np.float64) * c[None, :] * V) ** 2).sum()
    rhs = (hcol[None, :].astype(np.float64) * rho[:, None] * (Wp.astype(np.float64) - V) ** 2).sum()
    assert abs(lhs - rhs) <= 1e-5 * rhs


# --------------------------------------------------------------------------
def pin_init_walk(lib):
    """Seeding takes the first K bitwise-distinct sub-vectors in permutation
    order, as exact copies; repeats are skipped; too few distinct -> short."""
    g = np.random.default_rng(5)
    d = 4
    base = g.standard_normal((6, d)).astype(np.float32)
    X = base[[0, 1, 0, 2, 1, 3, 3, 4, 5, 0]]          # repeats at 2, 4, 6, 9
    perm = np.arange(10, dtype=np.int32)
    C, taken = O.init(X, d, perm, 6, lib)
    assert taken == 6
    assert np.array_equal(C.view(np.uint32), base[[0, 1, 2, 3, 4, 5]].view(np.uint32))
    perm = np.array([9, 8, 7, 6, 5, 4, 3, 2, 1, 0], np.int32)
    C, taken = O.init(X, d, perm, 4, lib)
    assert taken == 4
    assert np.array_equal(C.view(np.uint32), X[[9, 8, 7, 6]].view(np.uint32))
    C, taken = O.init(np.ones((50, d), np.float32), d, np.arange(50, dtype=np.int32), 3, lib)
    assert taken == 1
    # -0.0 and +0.0 are distinct bit patterns
    Z = np.array([[0.0, 0, 0, 0], [-0.0, 0, 0, 0]], np.float32)
    C, taken = O.init(Z, d, np.arange(2, dtype=np.int32), 2, lib)
    assert taken == 2


# --------------------------------------------------------------------------
def pin_assign_euclidean_special_case(lib):
    """h = 1, no mask, no row weight: the weighted search is Q_V of the VPTQ
    page's core algorithm, Euclidean nearest centroid -> scipy's vq."""
    g = np.random.default_rng(21)
    M, N, d, K = 16, 32, 8, 37
    X = g.standard_normal((M, N)).astype(np.float32)
    C = g.standard_normal((K, d)).astype(np.float32)
    idx, dist = O.assign(X, np.ones(N, np.float32), None, None, d, C, lib=lib)
    ref, rd = scvq.vq(X.reshape(-1, d).astype(np.float64), C.astype(np.float64))
    assert np.array_equal(idx, ref)
    assert np.allclose(dist, rd ** 2, rtol=1e-12)


def pin_assign_weighted_reduction(lib):
    """With per-element weights, D(s,k) is the squared Euclidean distance
    after scaling both sides by sqrt(omega_s); masked elements drop out.
    Checked per sub-vector against scipy's cdist, with several column blocks,
    a row weight and a mask; plus invariances (h -> 3h, centroid order)."""
    W, h, g = _case(9, 12, 40, n_ch=4)
    M, N = W.shape
    d, K = 8, 29
    C = (0.02 * g.standard_t(4, size=(K, d))).astype(np.float32)
    rho = g.uniform(0.5, 2.0, M).astype(np.float32)
    keep = (g.random((M, N)) > 0.15).astype(np.uint8)
    keep[3, 8:16] = 0                    # one fully masked sub-vector
    idx, dist = O.assign(W, h, rho, keep, d, C, lib=lib)
    nb = N // d
    for s in range(M * nb):
        i, b = divmod(s, nb)
        om = h[b * d:(b + 1) * d].astype(np.float64) * float(rho[i]) * keep[i, b * d:(b + 1) * d]
        sq = np.sqrt(om)
        dd = cdist((sq * W[i, b * d:(b + 1) * d])[None, :], sq[None, :] * C.astype(np.float64),
                   "sqeuclidean")[0]
        if s == 3 * nb + 1:
            assert np.all(dd == 0) and idx[s] == 0 and dist[s] == 0
            continue
        assert idx[s] == int(np.argmin(dd)), s
        assert abs(dist[s] - dd.min()) <= 1e-12 * max(dd.min(), 1e-300)
    idx3, _ = O.assign(W, 3.0 * h, rho, keep, d, C, lib=lib)
    assert np.array_equal(idx3, idx)
    perm = g.permutation(K)
    idxp, _ = O.assign(W, h, rho, keep, d, C[perm], lib=lib)
    live = np.ones(idx.size, bool)
    live[3 * nb + 1] = False             # all-zero distances: tie, lowest new index
    assert np.array_equal(perm[idxp][live], idx[live])


def pin_assign_tie_lowest(lib):
    """Equal distances go to the lowest centroid index."""
    g = np.random.default_rng(4)
    d = 8
    C = g.standard_normal((10, d)).astype(np.float32)
    C[7] = C[2]
    X = C[[2, 7, 2, 5]].reshape(1, -1)
    idx, _ = O.assign(X, np.ones(4 * d, np.float32), None, None, d, C, lib=lib)
    assert list(idx) == [2, 2, 2, 5]


def pin_assign_subset(lib):
    """Assigning a listed subset gives the same answers as the full pass."""
    W, h, g = _case(13, 10, 24)
    C = (0.02 * g.standard_t(4, size=(9, 8))).astype(np.float32)
    full, fd = O.assign(W, h, None, None, 8, C, lib=lib)
    sub = np.array([29, 0, 5, 17, 5], np.int64)
    part, pd = O.assign(W, h, None, None, 8, C, subset=sub, lib=lib)
    assert np.array_equal(part, full[sub]) and np.array_equal(pd, fd[sub])


# --------------------------------------------------------------------------
def pin_update_weighted_mean(lib):
    """The update is numpy's weighted average per (centroid, dimension) with
    weight omega; an empty centroid or a zero weight sum keeps its old value;
    counts are numpy's bincount; J is the objective of the input codebook
    (equal to the sum of the assigned distances)."""
    W, h, g = _case(17, 16, 48, n_ch=3)
    M, N = W.shape
    d, K = 8, 23
    C = (0.02 * g.standard_t(4, size=(K, d))).astype(np.float32)
    rho = g.uniform(0.5, 2.0, M).astype(np.float32)
    keep = (g.random((M, N)) > 0.2).astype(np.uint8)
    idx, dist = O.assign(W, h, rho, keep, d, C, lib=lib)
    idx = idx.copy()
    idx[idx == 4] = 3                       # centroid 4 left empty
    idx[idx == 11] = 12                     # centroid 11: one member, fully masked
    idx[7] = 11
    keep2 = keep.copy()
    i7, b7 = divmod(7, N // d)
    keep2[i7, b7 * d:(b7 + 1) * d] = 0
    Cn, counts, J = O.update(W, h, rho, keep2, d, idx, C, lib=lib)
    assert np.array_equal(counts, np.bincount(idx, minlength=K))
    X = W.reshape(-1, d).astype(np.float64)
    nb = N // d
    om = (h.reshape(nb, d)[None, :, :].astype(np.float64) * rho[:, None, None]
          * keep2.reshape(M, nb, d)).reshape(-1, d)
    for k in range(K):
        mem = idx == k
        for t in range(d):
            wsum = om[mem, t].sum()
            if wsum > 0:
                want = np.float32(np.average(X[mem, t], weights=om[mem, t]))
                assert abs(float(Cn[k, t]) - float(want)) <= 2e-7 * abs(float(want)) + 1e-30, (k, t)
            else:
                assert Cn[k, t] == C[k, t]
    assert np.array_equal(Cn[4], C[4]) and np.array_equal(Cn[11], C[11])
    Jref = (om * (X - C[idx].astype(np.float64)) ** 2).sum()
    assert abs(J - Jref) <= 1e-12 * Jref


def pin_update_optimality(lib):
    """Closed form: for fixed assignments the update is the exact minimizer of
    J, so moving any centroid component by +-delta never lowers J."""
    W, h, g = _case(19, 8, 32)
    d, K = 8, 6
    C = (0.02 * g.standard_t(4, size=(K, d))).astype(np.float32)
    idx, _ = O.assign(W, h, None, None, d, C, lib=lib)
    Cn, _, _ = O.update(W, h, None, None, d, idx, C, lib=lib)
    J0 = O.objective(W, h, None, None, d, Cn, idx, lib=lib)
    for k in range(K):
        for t in range(d):
            for delta in (1e-3, -1e-3):
                Cp = Cn.copy()
                Cp[k, t] += np.float32(delta * max(abs(float(Cn[k, t])), 1e-3))
                assert O.objective(W, h, None, None, d, Cp, idx, lib=lib) >= J0 * (1 - 1e-12)


# --------------------------------------------------------------------------
def pin_lloyd_matches_scipy_kmeans(lib):
    """h = 1, no mask, p = 0, one stage: T Lloyd iterations from a given
    codebook are scipy's kmeans2(minit='matrix', iter=T); the returned indices
    are scipy's vq of the final codebook (textbook Lloyd, as cited for K-means
    on the SCVQ page)."""
    g = np.random.default_rng(31)
    M, N, d, K, T = 64, 32, 8, 12, 6
    W = g.standard_normal((M, N)).astype(np.float32)
    perm = g.permutation(M * N // d).astype(np.int32)
    out = O.fit(W, np.ones(N, np.float32), d, K, T, 0, 0, 0.0, perm1=perm, lib=lib)
    X = W.reshape(-1, d).astype(np.float64)
    C0 = X[perm[:K]]
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        cb, _ = scvq.kmeans2(X, C0.copy(), iter=T, minit="matrix")
    assert np.allclose(out["C1"], cb, rtol=1e-5, atol=1e-6)
    lab, _ = scvq.vq(X, out["C1"].astype(np.float64))
    assert np.array_equal(out["idx1"], lab)


def pin_weighted_lloyd_reduces_to_scaled_kmeans(lib):
    """One column block (N = d), no row weight, no mask: weighted K-means on x
    with per-dimension weights h equals plain K-means on sqrt(h) * x, with
    centroids mapped back by 1/sqrt(h)."""
    g = np.random.default_rng(37)
    M, d, K, T = 300, 8, 10, 5
    W = g.standard_normal((M, d)).astype(np.float32)
    h = g.uniform(0.2, 5.0, d).astype(np.float32)
    perm = g.permutation(M).astype(np.int32)
    out = O.fit(W, h, d, K, T, 0, 0, 0.0, perm1=perm, lib=lib)
    sq = np.sqrt(h.astype(np.float64))
    Y = W.astype(np.float64) * sq
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        cb, _ = scvq.kmeans2(Y, Y[perm[:K]].copy(), iter=T, minit="matrix")
    assert np.allclose(out["C1"], cb / sq, rtol=1e-5, atol=1e-6)


def pin_fit_monotone_and_identity(lib):
    """Lloyd never raises J (both stages), and the last stage's final J equals
    the weighted error of the reconstructed matrix over the kept positions:
    sum_ij h_j keep_ij (W - What)_ij^2 (a real-arithmetic identity), while
    What == W bitwise at every salient position."""
    for binorm in (False, True):
        W, h, g = _case(41 + binorm, 32, 64, n_ch=3)
        M, N = W.shape
        d, K1, T1, K2, T2 = 8, 24, 6, 8, 4
        perm1 = g.permutation(M * N // d).astype(np.int32)
        perm2 = g.permutation(M * N // d).astype(np.int32)
        out = O.fit(W, h, d, K1, T1, K2, T2, 0.02, binorm=binorm, perm1=perm1, perm2=perm2, lib=lib)
        J = out["J"]
        for a, b in [(0, T1 + 1), (T1 + 1, T1 + T2 + 2)]:
            seg = J[a:b]
            assert np.all(seg[1:] <= seg[:-1] * (1 + 1e-12)), seg
        keep = out["keep"]
        err = (h[None, :].astype(np.float64) * keep * (W.astype(np.float64) - out["What"]) ** 2).sum()
        assert abs(err - J[-1]) <= 2e-5 * J[-1], (err, J[-1])
        sel = keep == 0
        assert np.array_equal(out["What"][sel].view(np.uint32), W[sel].view(np.uint32))
        assert sel.sum() == out["nnz"]


def _grouped_perms(g, M, layout):
    p1 = np.concatenate([g.permutation(M * Ng // dg) for _, Ng, dg, _, _, _, _ in layout]).astype(np.int32)
    p2 = [g.permutation(M * Ng // dg) for _, Ng, dg, _, _, K2g, _ in layout if K2g]
    return p1, (np.concatenate(p2).astype(np.int32) if p2 else np.zeros(1, np.int32))


def pin_grouped_reduces_to_fit(lib):
    """No outlier columns and one group: the grouped fit is the plain fit, bit for bit."""
    for binorm in (False, True):
        W, h, g = _case(51 + binorm, 24, 64, n_ch=3)
        M, N = W.shape
        d, K1, T1, K2, T2 = 8, 20, 4, 6, 3
        lay = O.grouped_layout(N, d, 0, 4, 0, 0, 1, K1, T1, K2, T2)
        p1, p2 = _grouped_perms(g, M, lay)
        gout = O.fit_grouped(W, h, d, K1, T1, K2, T2, 0.02, 0, 4, 0, 0, 1, p1, p2, binorm=binorm, lib=lib)
        out = O.fit(W, h, d, K1, T1, K2, T2, 0.02, binorm=binorm, perm1=p1, perm2=p2, lib=lib)
        n_sub = M * N // d
        assert np.array_equal(gout["cols"], np.arange(N, dtype=np.int32))
        assert np.array_equal(gout["idx"][:n_sub], out["idx1"]) and np.array_equal(gout["idx"][n_sub:], out["idx2"])
        assert np.array_equal(gout["cb"][:K1 * d], out["C1"].ravel())
        assert np.array_equal(gout["What"].view(np.uint32), out["What"].view(np.uint32))
        assert np.array_equal(gout["J"], out["J"])


def pin_grouped_columns_and_identity(lib):
    """The outlier group is the n_out columns with the largest h (ties: smaller index),
    listed ascending, then the rest ascending; every group's Lloyd stages never raise J;
    and the groups' final objectives add up to sum_ij h_j keep_ij (W - What)_ij^2 over
    the whole matrix (so every group's reconstruction landed in its own columns), with
    What == W at every salient position."""
    for binorm, n_groups in ((False, 2), (True, 3)):
        W, h, g = _case(53 + binorm, 24, 96, n_ch=4)
        h[5] = h[17] = h.max()                      # a tie at the top
        M, N = W.shape
        d, K1, T1, K2, T2, n_out, d0, K0, T0 = 8, 16, 4, 4, 3, 16, 4, 24, 5
        lay = O.grouped_layout(N, d, n_out, d0, K0, T0, n_groups, K1, T1, K2, T2)
        p1, p2 = _grouped_perms(g, M, lay)
        out = O.fit_grouped(W, h, d, K1, T1, K2, T2, 0.02, n_out, d0, K0, T0, n_groups, p1, p2, binorm=binorm,
                            lib=lib)
        order = np.lexsort((np.arange(N), -h.astype(np.float64)))
        top = np.sort(order[:n_out])
        rest = np.setdiff1d(np.arange(N), top)
        assert np.array_equal(out["cols"], np.concatenate([top, rest]).astype(np.int32))
        J, o, finals = out["J"], 0, []
        for _, Ng, dg, Kg, Tg, K2g, T2g in lay:
            segs = [Tg + 1] + ([T2g + 1] if K2g else [])
            for L in segs:
                seg = J[o:o + L]
                assert np.all(seg[1:] <= seg[:-1] * (1 + 1e-12)), seg
                o += L
            finals.append(J[o - 1])
        keep = out["keep"]
        err = (h[None, :].astype(np.float64) * keep * (W.astype(np.float64) - out["What"]) ** 2).sum()
        assert abs(err - sum(finals)) <= 2e-5 * sum(finals), (err, sum(finals))
        sel = keep == 0
        assert np.array_equal(out["What"][sel].view(np.uint32), W[sel].view(np.uint32))


def pin_degenerate_cases(lib):
    """K = n_sub with every sub-vector distinct: J = 0 and What == W bitwise.
    p = 1: every weight is held exactly, What == W and J = 0.  Residual
    decode: without scales, What = C1[i1] + C2[i2] at every kept position."""
    g = np.random.default_rng(43)
    M, N, d = 8, 16, 8
    W = (0.02 * g.standard_t(4, size=(M, N))).astype(np.float32)
    h = g.uniform(1, 5, N).astype(np.float32)
    n_sub = M * N // d
    perm = g.permutation(n_sub).astype(np.int32)
    out = O.fit(W, h, d, n_sub, 3, 0, 0, 0.0, perm1=perm, lib=lib)
    assert np.all(out["J"] == 0)
    assert np.array_equal(out["What"].view(np.uint32), W.view(np.uint32))
    out = O.fit(W, h, d, 4, 3, 2, 2, 1.0, perm1=perm, perm2=perm, lib=lib)
    assert np.all(out["J"] == 0)
    assert np.array_equal(out["What"].view(np.uint32), W.view(np.uint32))
    W2, h2, g2 = _case(47, 16, 32)
    p1 = g2.permutation(64).astype(np.int32)
    out = O.fit(W2, h2, 8, 10, 3, 6, 3, 0.0, perm1=p1, perm2=p1, lib=lib)
    dec = out["C1"][out["idx1"]] + out["C2"][out["idx2"]]
    assert np.array_equal(out["What"].reshape(-1, 8).view(np.uint32), dec.view(np.uint32))


def pin_fit_residual_seed(lib):
    """The residual stage seeds its codebook from the residual of the first
    stage (VPTQ page, "Residual Vector Quantization": the second codebook
    quantizes v - Q(v)): with no residual iterations, C2 holds the first K2
    distinct residual sub-vectors in perm2 order, bitwise."""
    W, h, g = _case(53, 16, 32)
    n_sub = 16 * 32 // 8
    p1 = g.permutation(n_sub).astype(np.int32)
    p2 = g.permutation(n_sub).astype(np.int32)
    out = O.fit(W, h, 8, 12, 2, 5, 0, 0.0, perm1=p1, perm2=p2, lib=lib)
    R = W.reshape(-1, 8) - out["C1"][out["idx1"]]
    seen, rows = set(), []
    for s in p2:
        key = R[s].tobytes()
        if key not in seen:
            seen.add(key)
            rows.append(R[s])
        if len(rows) == 5:
            break
    assert np.array_equal(out["C2"].view(np.uint32), np.array(rows).view(np.uint32))


def pin_bits_worked_example(lib):
    """The VPTQ page's compression-ratio example (golden fixture)."""
    import json
    import os
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "golden", "vptq_compression_example.json")) as f:
        ex = json.load(f)
    n = ex["matrix"][0] * ex["matrix"][1]
    cr = O.compression_ratio_single(n, ex["vector_length"], ex["centroids"],
                                    ex["original_bits"], ex["codebook_bits"])
    assert round(cr, ex["printed_ratio_decimals"]) == ex["printed_compression_ratio"]
    bpw = O.bits_per_weight(ex["matrix"][0], ex["matrix"][1], ex["vector_length"],
                            ex["centroids"], 0, 0, cb_bits=ex["codebook_bits"])
    assert round(bpw, ex["printed_bpw_decimals"]) == ex["printed_bits_per_weight"]
    assert abs(bpw - ex["original_bits"] / cr) < 1e-12


def pin_bits_grouped_counts(lib):
    """Grouped bits per weight: one group without outlier columns is the plain
    count; a two-group case counted by hand; splitting a group in two adds
    exactly one more set of codebooks."""
    for d, K1, K2, nnz, bn in [(8, 256, 0, 0, False), (8, 4096, 256, 37, True), (4, 16, 4, 5, False)]:
        a = O.bits_per_weight_grouped(32, 64, [(64, d, K1, K2)], nnz, 0, 32, bn)
        assert a == O.bits_per_weight(32, 64, d, K1, K2, nnz, 32, bn)
    # 16 x 24: outlier group 8 columns, v = 4, 16 centroids (32 sub-vectors x 4 bits,
    # 4 x 16 x 16 codebook bits); main group 16 columns, v = 8, 256 + 4 centroids
    # (32 sub-vectors x (8 + 2) bits, 8 x 260 x 16 codebook bits); 3 salient
    # entries (64 bits each + 17 row pointers); bi-norm 16 + 24 scales; 8 column ids.
    bits = 32 * 4 + 4 * 16 * 16 + 32 * 10 + 8 * 260 * 16 + 3 * 64 + 17 * 32 + 40 * 32 + 8 * 32
    assert O.bits_per_weight_grouped(16, 24, [(8, 4, 16, 0), (16, 8, 256, 4)], 3, 8, 16, True) == bits / 384
    one = O.bits_per_weight_grouped(64, 128, [(128, 8, 64, 8)], 0, 0, 32)
    two = O.bits_per_weight_grouped(64, 128, [(64, 8, 64, 8), (64, 8, 64, 8)], 0, 0, 32)
    assert (two - one) * 64 * 128 == 8 * (64 + 8) * 32


def _tie_case(seed, M, N):
    """Tiny matrix with many exact score ties: weights and h from small sets."""
    g = np.random.default_rng([13, seed])
    W = (g.integers(-3, 4, size=(M, N)) * 0.25).astype(np.float32)
    h = g.choice(np.array([0.5, 1.0, 2.0], np.float32), N)
    return W, h, g


def _subvector_scores_np(W, h, d):
    """fp32 score per sub-vector: sum over t in order of h_j * (w * w), numpy float32 ops."""
    M, N = W.shape
    Wr = W.reshape(M, N // d, d)
    hr = h.reshape(N // d, d)
    acc = np.zeros((M, N // d), np.float32)
    for t in range(d):
        term = (hr[None, :, t] * (Wr[:, :, t] * Wr[:, :, t])).astype(np.float32)
        acc = (acc + term).astype(np.float32)
    return acc.ravel()


def pin_select_subvectors_brute_force(lib):
    """Brute force with numpy: fp32 sub-vector scores, lexsort (score desc, id asc), and the
    selection ORed into an existing correction."""
    for seed, (M, N, d, n_sel) in enumerate([(6, 16, 4, 5), (5, 24, 8, 7), (4, 9, 3, 12), (3, 8, 8, 0)]):
        W, h, g = _tie_case(seed, M, N)
        n_sub = M * N // d
        sc = _subvector_scores_np(W, h, d)
        order = np.lexsort((np.arange(n_sub), -sc))
        keep0 = (g.random((M, N)) > 0.1).astype(np.uint8)
        exp = keep0.copy().reshape(n_sub, d)
        exp[order[:n_sel]] = 0
        got = O.select_subvectors(W, h, d, n_sel, keep=keep0, lib=lib)
        assert np.array_equal(got.reshape(n_sub, d), exp)
        # taking all sub-vectors clears everything
        assert not O.select_subvectors(W, h, d, n_sub, lib=lib).any()


def pin_select_residual_brute_force(lib):
    """Brute force with numpy over the kept positions only: fp32 h * (w - what)^2, lexsort
    (score desc, linear index asc); asking for more than remain takes every kept position."""
    for seed, (M, N, n_sel) in enumerate([(6, 16, 9), (5, 24, 30), (4, 10, 1000)]):
        W, h, g = _tie_case(seed + 10, M, N)
        What = (g.integers(-2, 3, size=(M, N)) * 0.25).astype(np.float32)
        keep0 = (g.random((M, N)) > 0.2).astype(np.uint8)
        r = (W - What).astype(np.float32)
        sc = (h[None, :] * (r * r).astype(np.float32)).astype(np.float32).ravel()
        lin = np.arange(M * N)
        cand = lin[keep0.ravel() == 1]
        order = cand[np.lexsort((cand, -sc[cand]))]
        exp = keep0.ravel().copy()
        exp[order[:n_sel]] = 0
        got = O.select_residual(W, What, h, n_sel, keep=keep0, lib=lib)
        assert np.array_equal(got.ravel(), exp)


def pin_keep_to_csr_matches_nonzero(lib):
    """The CSR of a mask is numpy's row-major nonzero list of the held positions."""
    W, h, g = _tie_case(20, 7, 13)
    keep = (g.random((7, 13)) > 0.3).astype(np.uint8)
    keep[2] = 1                                   # an empty row
    rp, col, val = O.keep_to_csr(W, keep, lib=lib)
    ii, jj = np.nonzero(keep == 0)
    assert np.array_equal(col, jj.astype(np.int32))
    assert np.array_equal(val, W[ii, jj])
    assert np.array_equal(rp, np.concatenate([[0], np.cumsum((keep == 0).sum(1))]).astype(np.int32))


def _vptq_case(seed, M=16, N=24, V=4, K=10, T=40):
    g = np.random.default_rng([17, seed])
    W = (0.05 * g.standard_t(4.0, size=(M, N))).astype(np.float32)
    X = g.standard_normal((T, N))
    X[:, g.choice(N, 2, replace=False)] *= 8.0
    H = X.T @ X
    C = (0.05 * g.standard_normal((K, V))).astype(np.float32)
    U = O.inverse_hessian_factor(H).astype(np.float32)
    return W, H, U, C


def pin_inverse_hessian_factor_properties(lib):
    """U is upper triangular with a positive diagonal and U^T U (H + damp mean(diag H) I) = I;
    for a diagonal H it is diag(1 / sqrt(h + damp mean h))."""
    g = np.random.default_rng(23)
    X = g.standard_normal((30, 12))
    H = X.T @ X
    U = O.inverse_hessian_factor(H, damp=0.01)
    Hd = H + 0.01 * np.mean(np.diag(H)) * np.eye(12)
    assert np.allclose(np.tril(U, -1), 0.0) and np.all(np.diag(U) > 0)
    assert np.allclose(U.T @ U @ Hd, np.eye(12), atol=1e-10)
    h = g.uniform(1.0, 3.0, 7)
    U2 = O.inverse_hessian_factor(np.diag(h), damp=0.1)
    assert np.allclose(U2, np.diag(1.0 / np.sqrt(h + 0.1 * h.mean())), rtol=1e-14)


def pin_vptq_error_factorization(lib):
    """Algorithm 1's updates leave W - What = E U exactly (each column's final
    error is its own scaled error plus everything pushed into it from the left),
    for any upper-triangular U; and with GPTQ's U the OBS objective
    tr(dW H dW^T) is ||E||^2 up to the damping (here within 5%)."""
    W, H, U, C = _vptq_case(1)
    for B in (5, 24):
        idx, What, E, gap = O.vptq(W, U, 4, C, B, lib=lib)
        dW = W.astype(np.float64) - What.astype(np.float64)
        assert np.allclose(dW, E @ U.astype(np.float64), rtol=1e-10, atol=1e-12)
        obj = float(np.trace(dW @ H @ dW.T))
        assert abs(obj - float((E * E).sum())) <= 0.05 * obj


def pin_vptq_quantizes_updated_columns(lib):
    """Each column's indices are scipy's Euclidean nearest codebook rows of that
    column as updated by every error to its left: W[:,n] - sum_{n'<n} E[:,n'] U[n',n]."""
    W, H, U, C = _vptq_case(2)
    V = 4
    idx, What, E, gap = O.vptq(W, U, V, C, 7, lib=lib)
    M, N = W.shape
    Ud = U.astype(np.float64)
    for n in range(N):
        wn = W[:, n].astype(np.float64) - E[:, :n] @ Ud[:n, n]
        ref, _ = scvq.vq(wn.reshape(M // V, V), C.astype(np.float64))
        ok = gap[n] > 1e-9
        assert np.array_equal(idx[n][ok], ref[ok].astype(np.uint16))
        assert np.array_equal(What[:, n], C[idx[n]].ravel())


def pin_vptq_block_size_invariance(lib):
    """Deferring the pushes to columns past the block (the block-boundary update)
    changes nothing in exact arithmetic: B = 1, 3 and N agree."""
    W, H, U, C = _vptq_case(3)
    runs = [O.vptq(W, U, 4, C, B, lib=lib) for B in (1, 3, W.shape[1])]
    for idx, What, E, gap in runs[1:]:
        ok = (gap > 1e-9) & (runs[0][3] > 1e-9)
        assert np.array_equal(idx[ok], runs[0][0][ok])
        assert np.allclose(E, runs[0][2], rtol=1e-9, atol=1e-12)


def pin_vptq_identity_is_plain_vq(lib):
    """With U = I there is no coupling: every column is plain Euclidean VQ of the
    original weights and E = W - What."""
    W, H, U, C = _vptq_case(4)
    M, N = W.shape
    idx, What, E, gap = O.vptq(W, np.eye(N, dtype=np.float32), 4, C, 5, lib=lib)
    for n in range(N):
        ref, _ = scvq.vq(W[:, n].astype(np.float64).reshape(M // 4, 4), C.astype(np.float64))
        assert np.array_equal(idx[n], ref.astype(np.uint16))
    assert np.array_equal(E, W.astype(np.float64) - What.astype(np.float64))


def _qg_case(seed, M=6, N=24, d=4, K1=7, K2=3, B=3, pow2_scales=False):
    g = np.random.default_rng([11, seed])
    nb = N // d
    C1 = g.standard_normal((K1, d)).astype(np.float32)
    C2 = (0.1 * g.standard_normal((K2, d))).astype(np.float32)
    idx1 = g.integers(0, K1, M * nb).astype(np.uint16)
    idx2 = g.integers(0, K2, M * nb).astype(np.uint16)
    if pow2_scales:
        r = np.ldexp(1.0, g.integers(-3, 4, M)).astype(np.float32)
        c = np.ldexp(1.0, g.integers(-3, 4, N)).astype(np.float32)
    else:
        r = g.uniform(0.5, 2.0, M).astype(np.float32)
        c = g.uniform(0.5, 2.0, N).astype(np.float32)
    # two salient positions in row 1, none in row 0, one in the last row
    rows = {1: [3, N - 1], M - 1: [0]}
    row_ptr = np.zeros(M + 1, np.int32)
    col, val = [], []
    for i in range(M):
        for j in rows.get(i, []):
            col.append(j)
            val.append(g.standard_normal() * 5.0)
        row_ptr[i + 1] = len(col)
    X = g.standard_normal((B, N)).astype(np.float32)
    return dict(M=M, N=N, d=d, C1=C1, idx1=idx1, C2=C2, idx2=idx2, r=r, c=c, row_ptr=row_ptr,
                col=np.array(col, np.int32), val=np.array(val, np.float32)), X


def pin_qgemv_unit_tokens(lib):
    """Multiplying by the unit vectors e_j reads back column j of the
    reconstruction, for every token row: pins rows, columns and the token
    stride of the product to the (separately pinned) reconstruction."""
    cs, _ = _qg_case(1)
    N = cs["N"]
    What = O.reconstruct(lib=lib, **cs)
    Y = O.qgemv(X=np.eye(N, dtype=np.float32), lib=lib, **cs)
    assert Y.shape == (N, cs["M"])
    assert np.array_equal(Y, What.T.astype(np.float64))


def pin_qgemv_matches_numpy_matmul(lib):
    """Special case of a library routine: numpy's float64 matrix product of the
    reconstruction with the activations."""
    cs, X = _qg_case(2, M=9, N=40, d=8, B=4)
    What = O.reconstruct(lib=lib, **cs).astype(np.float64)
    ref = X.astype(np.float64) @ What.T
    Y = O.qgemv(X=X, lib=lib, **cs)
    assert np.allclose(Y, ref, rtol=1e-13, atol=1e-13)


def pin_qgemv_power_of_two_scales(lib):
    """With power-of-two row and column scales, What(r, c) = r_i * What(1, 1) * c_j
    exactly, so Y(r, c; X) = r * Y(1, 1; X * c) bit for bit (rows scale outputs,
    columns scale inputs)."""
    cs, X = _qg_case(3, pow2_scales=True)
    cs["row_ptr"] = cs["col"] = cs["val"] = None
    r, c = cs.pop("r"), cs.pop("c")
    Y = O.qgemv(X=X, r=r, c=c, lib=lib, **cs)
    Y1 = O.qgemv(X=X * c[None, :], lib=lib, **cs)
    assert np.array_equal(Y, Y1 * r[None, :].astype(np.float64))


def pin_qgemv_float64_accumulation(lib):
    """A row [2^30, 1, -2^30, 0, ...] against ones gives exactly 1; a float32
    running sum would return 0."""
    d, N = 4, 8
    C1 = np.array([[2.0 ** 30, 1.0, -(2.0 ** 30), 0.0], [0.0, 0.0, 0.0, 0.0]], np.float32)
    idx1 = np.array([0, 1], np.uint16)
    Y = O.qgemv(1, N, d, C1, idx1, np.ones((1, N), np.float32), lib=lib)
    assert Y[0, 0] == 1.0


def pin_qgemv_sparse_term(lib):
    """The salient positions replace the decoded weight: adding the CSR changes
    y_i by sum_k (val_k - What_dense[i, col_k]) * x[col_k], and rows without
    salient positions do not change at all."""
    cs, X = _qg_case(4)
    Y = O.qgemv(X=X, lib=lib, **cs)
    dense = dict(cs, row_ptr=None, col=None, val=None)
    Y0 = O.qgemv(X=X, lib=lib, **dense)
    Wd = O.reconstruct(lib=lib, **dense).astype(np.float64)
    rp, col, val = cs["row_ptr"], cs["col"], cs["val"]
    for i in range(cs["M"]):
        e = list(range(rp[i], rp[i + 1]))
        if not e:
            assert np.array_equal(Y[:, i], Y0[:, i])
            continue
        delta = sum((float(val[k]) - Wd[i, col[k]]) * X[:, col[k]].astype(np.float64) for k in e)
        assert np.allclose(Y[:, i] - Y0[:, i], delta, rtol=1e-12, atol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
