"""Seeded input generation (CPU only)."""
import numpy as np
import torch

from hessian_weighted_vector_amd import configs, synth


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(3)
    x = (g.standard_normal(100000) * np.exp(g.standard_normal(100000) * 3)).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # exact ties
    ours = synth.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_generator_is_deterministic_and_shaped():
    cfg = configs.get(1)
    a = synth.make_inputs(cfg)
    b = synth.make_inputs(cfg)
    for k in ("W", "h", "perm1", "perm2"):
        assert synth.sha256(a[k]) == synth.sha256(b[k])
    assert a["W"].shape == (cfg.M, cfg.N) and a["W"].dtype == np.float32
    assert a["h"].shape == (cfg.N,) and np.all(a["h"] > 0)
    assert np.array_equal(np.sort(a["perm1"]), np.arange(cfg.n_sub))
    # the chosen high-energy channels carry the largest Hessian diagonal entries
    top = np.argsort(-a["h"])[:cfg.n_ch]
    assert set(top.tolist()) == set(a["channels"].tolist())


def test_config_table():
    sizes = [(c.M, c.N, c.K1, c.K2) for c in configs.CONFIGS]
    assert sizes == [(256, 256, 256, 0), (2048, 2048, 4096, 256), (8192, 2048, 65536, 256),
                     (4096, 11008, 65536, 256), (8192, 28672, 65536, 4096)]
    assert [c.n_sub for c in configs.CONFIGS] == [8192, 524288, 2097152, 5636096, 29360128]
