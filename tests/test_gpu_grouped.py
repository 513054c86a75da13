"""Parity of the grouped fit (outlier columns with their own codebook, the other
columns in independent groups) with the oracle (GPU).

Bar (as for the plain fit): CSR, masks and the column order bit for bit;
every group's indices bit for bit; codebooks within 1e-5 of each centroid's
max norm; objectives within 1e-5 relative; and the reconstruction bit for bit
when the trajectories agree.  The 4096 x 11008 workload (1% outlier columns,
v0 = 4, k0 = 4096) is checked against the properties that define it: the
column order against the oracle's, every group's objective never rising, the
groups' final objectives adding up to the whole matrix's weighted error, and
the salient values held exactly.
"""
import sys

import numpy as np
import pytest

import oracle
from gpu_util import bits_equal, centroid_close, dev, host, mask_from_keep
from hessian_weighted_vector_amd import configs, synth, vq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def perms(seed, M, layout):
    g = np.random.default_rng([81, seed])
    p1 = np.concatenate([g.permutation(M * Ng // dg) for _, Ng, dg, _, _, _, _ in layout]).astype(np.int32)
    p2 = [g.permutation(M * Ng // dg) for _, Ng, dg, _, _, K2g, _ in layout if K2g]
    return p1, (np.concatenate(p2).astype(np.int32) if p2 else np.zeros(1, np.int32))


def run_both(W, h, d, K1, T1, K2, T2, p, binorm, n_out, d0, K0, T0, ng, seed, mask_outliers=True):
    M, N = W.shape
    lay = oracle.grouped_layout(N, d, n_out, d0, K0, T0, ng, K1, T1, K2, T2)
    p1, p2 = perms(seed, M, lay)
    o = oracle.fit_grouped(W, h, d, K1, T1, K2, T2, p, n_out, d0, K0, T0, ng, p1, p2, binorm=binorm,
                           mask_outliers=mask_outliers)
    prm = vq.grouped_params(M, N, d, K1, T1, K2, T2, p, binorm, mask_outliers, n_out, d0, K0, T0, ng)
    g = vq.fit_grouped(dev(W), dev(h), prm, p1, p2)
    return o, g, lay


def compare(o, g, lay, M, d):
    assert bits_equal(host(g["cols"]), o["cols"])
    assert bits_equal(host(g["row_ptr"]), o["row_ptr"])
    assert bits_equal(host(g["col"]), o["col"])
    assert bits_equal(host(g["val"]), o["val"])
    assert bits_equal(host(g["mask"]), mask_from_keep(o["keep"], d))
    assert bits_equal(host(g["idx"])[:o["idx"].size], o["idx"])
    cb = host(g["codebooks"])
    oc = 0
    for _, Ng, dg, Kg, _, K2g, _ in lay:
        for K in ([Kg, K2g] if K2g else [Kg]):
            ok, bad = centroid_close(cb[oc:oc + K * dg].reshape(K, dg), o["cb"][oc:oc + K * dg].reshape(K, dg))
            assert ok, bad[:10]
            oc += K * dg
    assert np.allclose(g["J"], o["J"], rtol=1e-5, atol=0)
    return bits_equal(host(g["W_hat"]), o["What"])


@pytest.mark.parametrize("binorm,ng", [(False, 2), (True, 3)])
def test_grouped_tiny_config_matches_oracle(binorm, ng):
    cfg = configs.get(1)
    say("grouped", cfg.name, "binorm", binorm, "groups", ng)
    inp = synth.make_inputs(cfg)
    o, g, lay = run_both(inp["W"], inp["h"], cfg.d, cfg.K1, cfg.T1, 32, 4, cfg.p, binorm, 16, 4, 64, 5, ng, 1)
    assert compare(o, g, lay, cfg.M, cfg.d)
    assert g["bpw"] == pytest.approx(oracle.bits_per_weight_grouped(
        cfg.M, cfg.N, [(Ng, dg, Kg, K2g) for _, Ng, dg, Kg, _, K2g, _ in lay], oracle.nnz(cfg.M, cfg.N, cfg.p),
        16, 32, binorm))


def test_grouped_without_groups_is_the_plain_fit():
    """n_out = 0 and one group: the grouped fit equals vq_fit bit for bit."""
    say("grouped = plain")
    inp = synth.small_case(91, 48, 64, d=8)
    W, h = inp["W"], inp["h"]
    o, g, lay = run_both(W, h, 8, 24, 4, 6, 3, 0.03, False, 0, 4, 0, 0, 1, 2)
    assert compare(o, g, lay, 48, 8)
    p1, p2 = perms(2, 48, lay)
    f = vq.fit(dev(W), dev(h), 8, 24, 4, 6, 3, 0.03, False, True, p1, p2)
    assert bits_equal(host(f["W_hat"]), host(g["W_hat"]))
    assert bits_equal(host(f["idx1"]), host(g["idx"])[:384])


def test_grouped_edge_cases():
    """d0 = 2, the outlier group only needing one stage, an unmasked fit, a
    last main group narrower than the others, K = n_sub in the outlier group."""
    say("grouped edge cases")
    inp = synth.small_case(92, 32, 88, d=8)
    W, h = inp["W"], inp["h"]
    # n_out = 8, d0 = 2: outlier group 32 x 8 -> 128 sub-vectors, K0 = 128 = n_sub
    o, g, lay = run_both(W, h, 8, 16, 3, 0, 0, 0.02, False, 8, 2, 128, 2, 3, 3, mask_outliers=False)
    assert [x[1] for x in lay] == [8, 32, 32, 16]
    assert compare(o, g, lay, 32, 8)


def test_grouped_smollm2_config_matches_oracle():
    """The 2048 x 2048 workload with 24 outlier columns (v0 = 4, k0 = 512) and
    two main groups."""
    cfg = configs.get(2)
    say("grouped", cfg.name)
    inp = synth.make_inputs(cfg)
    o, g, lay = run_both(inp["W"], inp["h"], cfg.d, cfg.K1, cfg.T1, cfg.K2, cfg.T2, cfg.p, cfg.binorm, 24, 4, 512,
                         cfg.T1, 2, 4)
    assert compare(o, g, lay, cfg.M, cfg.d)


def test_grouped_fullsize_properties():
    cfg = configs.get(4)
    say("grouped full size", cfg.name)
    inp = synth.make_inputs(cfg)
    W, h = inp["W"], inp["h"]
    M, N, d = cfg.M, cfg.N, cfg.d
    n_out = int(0.01 * N) // 8 * 8
    lay = oracle.grouped_layout(N, d, n_out, 4, 4096, cfg.T1, 1, cfg.K1, cfg.T1, cfg.K2, cfg.T2)
    p1, p2 = perms(5, M, lay)
    prm = vq.grouped_params(M, N, d, cfg.K1, cfg.T1, cfg.K2, cfg.T2, cfg.p, cfg.binorm, True, n_out, 4, 4096,
                            cfg.T1, 1)
    g = vq.fit_grouped(dev(W), dev(h), prm, p1, p2)
    assert bits_equal(host(g["cols"]), oracle.column_order(h, n_out))
    J, o_, finals = g["J"], 0, []
    for _, Ng, dg, Kg, Tg, K2g, T2g in lay:
        for L in [Tg + 1] + ([T2g + 1] if K2g else []):
            seg = J[o_:o_ + L]
            assert np.all(seg[1:] <= seg[:-1] * (1 + 1e-6)), seg
            o_ += L
        finals.append(J[o_ - 1])
    keep = 1 - np.unpackbits(host(g["mask"])[:, None], axis=1, bitorder="little").reshape(M, N)
    What = host(g["W_hat"])
    err = (h[None, :].astype(np.float64) * keep * (W.astype(np.float64) - What) ** 2).sum()
    say("  sum of group objectives %.6g, weighted error %.6g" % (sum(finals), err))
    assert abs(err - sum(finals)) <= 1e-4 * sum(finals)
    sel = keep == 0
    assert sel.sum() == oracle.nnz(M, N, cfg.p)
    assert np.array_equal(What[sel].view(np.uint32), W[sel].view(np.uint32))
