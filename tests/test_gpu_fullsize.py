"""Parity at the full workload sizes, in the launch configuration the
benchmark times (GPU).

The oracle cannot assign millions of sub-vectors against 65536 centroids
in test time, so:
  * assignment: every sub-vector is assigned on the GPU and a seeded sample
    of them (including salient-masked ones) is assigned by the oracle;
    indices must match bit for bit, distances to float32 rounding;
  * update, residual, objective and reconstruction run in full on both sides
    with seeded synthetic indices and CSR (inputs never come from the GPU);
  * selection is checked against the properties that define it (count,
    threshold, tie order, exact values, CSR structure) on every element;
  * the whole fit is checked for a non-increasing objective and for the
    identity J_final == sum_ij h_j keep_ij (W - What)_ij^2.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import bits_equal, centroid_close, check_select_properties, dev, host, keep_from_mask, mask_from_keep
from hessian_weighted_vector_amd import configs, synth, vq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", params=[3, 4, 5], ids=["mlp-up-8192x2048", "llama2-7b-4096x11008",
                                                       "70b-mlp-8192x28672"])
def world(request):
    cfg = configs.get(request.param)
    say("generating", cfg.name)
    inp = synth.make_inputs(cfg)
    W, h = inp["W"], inp["h"]
    if cfg.binorm:
        Wp, r, c, hcol, rho = oracle.binorm(W, h)
    else:
        Wp, r, c, hcol, rho = W, None, None, h, None
    nnz = oracle.nnz(cfg.M, cfg.N, cfg.p)
    ws = vq.workspace(cfg.M, cfg.N, cfg.d, cfg.K1, cfg.K2, nnz)
    g = np.random.default_rng([cfg.cid, 77])
    w = dict(cfg=cfg, inp=inp, W=W, h=h, Wp=Wp, r=r, c=c, hcol=hcol, rho=rho, nnz=nnz, ws=ws, g=g)
    yield w
    del w
    torch.cuda.empty_cache()


def test_binorm_fullsize(world):
    cfg = world["cfg"]
    if not cfg.binorm:
        pytest.skip("workload is not bi-normalized")
    say("binorm", cfg.name)
    got = [host(t) for t in vq.binorm(dev(world["W"]), dev(world["h"]), world["ws"])]
    ref = [world["Wp"], world["r"], world["c"], world["hcol"], world["rho"]]
    for a, b in zip(got, ref):
        ulp = np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))
        assert ulp.max() <= 1
        assert (ulp > 0).mean() < 1e-4


def test_select_fullsize_properties(world):
    cfg, W, h, nnz = world["cfg"], world["W"], world["h"], world["nnz"]
    say("select", cfg.name, "nnz", nnz)
    rp, col, val, mask = [host(t) for t in vq.sparse_select(dev(W), dev(h), cfg.d, nnz, world["ws"])]
    check_select_properties(W, h, cfg.d, nnz, rp, col, val, mask)


def test_init_and_sampled_assign_fullsize(world):
    cfg, Wp, hcol, rho = world["cfg"], world["Wp"], world["hcol"], world["rho"]
    say("init + assign", cfg.name)
    C, taken = oracle.init(Wp, cfg.d, world["inp"]["perm1"], cfg.K1)
    assert taken == cfg.K1
    Cg = vq.init(dev(Wp), cfg.d, world["inp"]["perm1"], cfg.K1, world["ws"])
    assert bits_equal(host(Cg), C)
    # a seeded mask with salient positions concentrated in the high-energy columns
    M, N = Wp.shape
    keep = np.ones((M, N), np.uint8)
    ch = world["inp"]["channels"]
    rows = world["g"].integers(0, M, size=4096)
    keep[rows[:, None], ch[None, : min(len(ch), 8)]] = 0
    mask = mask_from_keep(keep, cfg.d)
    idx, dist = vq.assign(dev(Wp), dev(hcol), None if rho is None else dev(rho), dev(mask), cfg.d, Cg,
                          world["ws"], want_dist=True)
    n_exact = vq.assign_exact_count(world["ws"], cfg.n_sub, cfg.K1)
    gi, gd = host(idx), host(dist)
    say("  exact re-searches:", n_exact, "of", cfg.n_sub)
    masked_ids = np.flatnonzero(mask)
    sample = np.unique(np.concatenate([world["g"].choice(cfg.n_sub, 1536, replace=False),
                                       world["g"].choice(masked_ids, min(512, masked_ids.size), replace=False)]))
    ref_idx, ref_d = oracle.assign(Wp, hcol, rho, keep, cfg.d, C, subset=sample.astype(np.int64))
    assert bits_equal(gi[sample], ref_idx), np.flatnonzero(gi[sample] != ref_idx)[:10]
    assert bits_equal(gd[sample], ref_d.astype(np.float32))
    assert n_exact < 0.05 * cfg.n_sub


def _synthetic_indices(world, K):
    return world["g"].integers(0, K, size=world["cfg"].n_sub).astype(np.uint16)


@pytest.mark.parametrize("stage", [1, 2])
def test_update_and_objective_fullsize(world, stage):
    cfg, Wp, hcol, rho = world["cfg"], world["Wp"], world["hcol"], world["rho"]
    K = cfg.K1 if stage == 1 else cfg.K2
    say("update", cfg.name, "K", K)
    C, _ = oracle.init(Wp, cfg.d, world["inp"]["perm2"], K)
    idx = _synthetic_indices(world, K)
    idx[: K // 2] = np.arange(K // 2)           # every other centroid surely non-empty
    M, N = Wp.shape
    keep = np.ones((M, N), np.uint8)
    keep[:, world["inp"]["channels"]] = 0        # salient columns excluded
    Cref, cref, Jref = oracle.update(Wp, hcol, rho, keep, cfg.d, idx, C)
    Cg = dev(C)
    counts, J = vq.update(dev(Wp), dev(hcol), None if rho is None else dev(rho), dev(mask_from_keep(keep, cfg.d)),
                          cfg.d, dev(idx), Cg, world["ws"])
    ok, bad = centroid_close(host(Cg), Cref)
    assert ok, bad[:10]
    assert np.array_equal(host(counts), cref)
    assert abs(float(host(J)[0]) - Jref) <= 1e-10 * abs(Jref)


def test_residual_reconstruct_fullsize(world):
    cfg, Wp, W = world["cfg"], world["Wp"], world["W"]
    say("residual + reconstruct", cfg.name)
    M, N = Wp.shape
    K2 = cfg.K2 or 1
    C1, _ = oracle.init(Wp, cfg.d, world["inp"]["perm1"], 4096)
    i1 = _synthetic_indices(world, 4096)
    R = oracle.residual(Wp, cfg.d, C1, i1)
    assert bits_equal(host(vq.residual(dev(Wp), cfg.d, dev(C1), dev(i1))), R)
    C2, _ = oracle.init(R, cfg.d, world["inp"]["perm2"], K2)
    i2 = _synthetic_indices(world, K2)
    # a seeded CSR: up to 8 positions per row, exact W values
    g = world["g"]
    per = g.integers(0, 9, size=M)
    rp = np.concatenate([[0], np.cumsum(per)]).astype(np.int32)
    col = np.concatenate([np.sort(g.choice(N, k, replace=False)) for k in per]).astype(np.int32)
    rows = np.repeat(np.arange(M), per)
    val = W[rows, col].copy()
    ref = oracle.reconstruct(M, N, cfg.d, C1, i1, C2, i2, world["r"], world["c"], rp, col, val)
    got = vq.reconstruct(M, N, cfg.d, dev(C1), dev(i1), dev(C2), dev(i2),
                         None if world["r"] is None else dev(world["r"]),
                         None if world["c"] is None else dev(world["c"]), dev(rp), dev(col), dev(val))
    assert bits_equal(host(got), ref)


@pytest.mark.parametrize("B", [1, 8])
def test_qgemv_fullsize(world, B):
    """The fused product at the full shape with the full codebook sizes and a
    seeded ~1% CSR, every output against the oracle within the header's bound
    (one token: the decode shape the benchmark times; eight: a batched decode)."""
    cfg, Wp = world["cfg"], world["Wp"]
    M, N, d = cfg.M, cfg.N, cfg.d
    say("qgemv", cfg.name, "B =", B)
    g = np.random.default_rng([cfg.cid, 91, B])
    n_sub = M * N // d
    flat = Wp.reshape(-1, d)
    C1 = flat[np.sort(g.choice(n_sub, cfg.K1, replace=False))].copy()
    K2 = cfg.K2 or 1
    C2 = (0.1 * flat[np.sort(g.choice(n_sub, K2, replace=False))]).astype(np.float32)
    i1 = g.integers(0, cfg.K1, n_sub).astype(np.uint16)
    i2 = g.integers(0, K2, n_sub).astype(np.uint16)
    per = g.integers(0, int(2 * cfg.p * N) + 1, size=M)
    rp = np.concatenate([[0], np.cumsum(per)]).astype(np.int32)
    col = np.concatenate([np.sort(g.choice(N, k, replace=False)) for k in per]).astype(np.int32)
    rows = np.repeat(np.arange(M), per)
    val = world["W"][rows, col].copy()
    X = g.standard_normal((B, N)).astype(np.float32)
    r, c = world["r"], world["c"]
    ref = oracle.qgemv(M, N, d, C1, i1, X, C2, i2, r, c, rp, col, val)
    Wd = np.abs(oracle.reconstruct(M, N, d, C1, i1, C2, i2, r, c).astype(np.float64))
    Xa = np.abs(X.astype(np.float64))
    T = Xa @ Wd.T
    extra = np.zeros((B, M))
    np.add.at(extra.T, rows, ((Wd[rows, col] + np.abs(val.astype(np.float64)))[:, None] * Xa[:, col].T))
    T += extra
    del Wd
    tol = (N / 32.0 + per[None, :].astype(np.float64) + 40.0) * 2.0 ** -24 * T
    got = vq.qgemv(M, N, d, dev(C1), dev(i1), dev(X), dev(C2), dev(i2),
                   None if r is None else dev(r), None if c is None else dev(c), dev(rp), dev(col), dev(val))
    err = np.abs(host(got).astype(np.float64) - ref)
    say("  max err / bound = %.3g" % float((err / tol).max()))
    assert np.all(err <= tol)


def test_fit_fullsize_properties(world):
    cfg, W, h = world["cfg"], world["W"], world["h"]
    say("fit", cfg.name)
    inp = world["inp"]
    out = vq.fit(dev(W), dev(h), cfg.d, cfg.K1, cfg.T1, cfg.K2, cfg.T2, cfg.p, cfg.binorm, True,
                 inp["perm1"], inp["perm2"], ws=world["ws"])
    J = out["J"]
    say("  J:", J[0], "->", J[cfg.T1], "|", J[cfg.T1 + 1], "->", J[-1])
    for a, b in [(0, cfg.T1 + 1), (cfg.T1 + 1, len(J))]:
        seg = J[a:b]
        assert np.all(seg[1:] <= seg[:-1] * (1 + 1e-6)), seg
    What = host(out["W_hat"])
    keep = keep_from_mask(host(out["mask"]), cfg.M, cfg.N, cfg.d)
    err = (h[None, :].astype(np.float64) * keep * (W.astype(np.float64) - What) ** 2).sum()
    assert abs(err - J[-1]) <= 1e-5 * J[-1], (err, J[-1])
    sel = keep == 0
    assert bits_equal(What[sel], W[sel])
    assert out["bpw"] == pytest.approx(oracle.bits_per_weight(cfg.M, cfg.N, cfg.d, cfg.K1, cfg.K2,
                                                              world["nnz"], 32, cfg.binorm))
