"""Seeded synthetic inputs shared by the GPU path's callers and the oracle's tests.

This module holds only input construction: random draws, the bfloat16
rounding of the input weights, and the activation energy that plays the role
of the Hessian diagonal.  None of the quantization method's arithmetic lives
here.

Recipe (stand-in for real LLM weights and calibration activations):
  * W = scale * StudentT(nu), shape [M, N] (out x in), float64 -> float32;
    heavy tails as the HAS-VQ abstract describes LLM weight distributions.
    For bf16 workloads W is rounded to bfloat16 (nearest-even) and held as fp32.
  * X = N(0, 1), shape [T, N]; n_ch distinct channels are multiplied by a gain,
    giving the few high-energy input channels that the VPTQ page ("Outlier
    Elimination") says show up as large Hessian diagonal entries.
  * h_j = sum_t X[t, j]^2 (accumulated in float64, stored fp32): the diagonal of
    X^T X, i.e. the diagonal Hessian proxy of a linear layer's input; the full
    H = X^T X (make_hessian) for the second-order error propagation.
  * perm1, perm2: seeded permutations of the sub-vector ids (codebook seeding).
Streams: rng([cid, s]) with s = 0 W, 1 X, 2 channel choice, 3 perm1, 4 perm2.
"""
import hashlib

import numpy as np


def rng(cid: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(cid), int(stream)])


def round_bf16(a32: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 (round to nearest, ties to even) -> exact fp32."""
    b = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def make_weight(cid, M, N, scale, nu, bf16):
    w = (scale * rng(cid, 0).standard_t(nu, size=(M, N))).astype(np.float32)
    return round_bf16(w) if bf16 else w


def make_activations(cid, N, T, n_ch, gain):
    """The synthetic calibration activations X [T x N] (float64) and the
    high-energy channels."""
    X = rng(cid, 1).standard_normal((T, N))
    ch = rng(cid, 2).choice(N, n_ch, replace=False)
    X[:, ch] *= gain
    return X, np.sort(ch)


def make_hdiag(cid, N, T, n_ch, gain):
    X, ch = make_activations(cid, N, T, n_ch, gain)
    return np.einsum("tj,tj->j", X, X).astype(np.float32), ch


def make_hessian(cid, N, T, n_ch, gain):
    """The full Hessian proxy H = X^T X [N x N] of a linear layer's input
    (float64 products and sums, stored fp32); its diagonal is make_hdiag's h
    up to the order of the float64 sums."""
    X, _ = make_activations(cid, N, T, n_ch, gain)
    return (X.T @ X).astype(np.float32)


def make_perm(cid, stream, n_sub):
    return rng(cid, stream).permutation(n_sub).astype(np.int32)


def make_inputs(cfg):
    """All inputs of one workload as numpy arrays (host memory)."""
    W = make_weight(cfg.cid, cfg.M, cfg.N, cfg.scale, cfg.nu, cfg.bf16)
    h, ch = make_hdiag(cfg.cid, cfg.N, cfg.T, cfg.n_ch, cfg.ch_gain)
    n_sub = cfg.M * cfg.N // cfg.d
    return {
        "W": W,
        "h": h,
        "channels": ch,
        "perm1": make_perm(cfg.cid, 3, n_sub),
        "perm2": make_perm(cfg.cid, 4, n_sub),
    }


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def small_case(seed, M, N, d=8, K=16, scale=0.02, nu=4.0, n_ch=2, gain=20.0, T=64):
    """A small seeded case of arbitrary shape for unit and parity tests."""
    g = np.random.default_rng([1000 + int(seed), 0])
    W = (scale * g.standard_t(nu, size=(M, N))).astype(np.float32)
    X = g.standard_normal((T, N))
    ch = g.choice(N, min(n_ch, N), replace=False)
    X[:, ch] *= gain
    h = np.einsum("tj,tj->j", X, X).astype(np.float32)
    n_sub = M * N // d
    return {"W": W, "h": h, "perm1": g.permutation(n_sub).astype(np.int32),
            "perm2": g.permutation(n_sub).astype(np.int32)}
