"""The allocation-free assignment entry point (vq_assign_noalloc) against
vq_assign with a caller workspace, through the C ABI (GPU).

The two must agree bit for bit (indices and distances) on consecutive calls
that share the library's device scratch array: a long-codebook call with
salient masks and row weights, then a smaller short-codebook one, then the
long one again.  Sizes beyond the array are rejected before any launch.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import bits_equal, dev, host, keep_from_mask, mask_from_keep
from hessian_weighted_vector_amd import synth, vq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(seed, M, N, d, K, p=0.02):
    g = np.random.default_rng([123, seed])
    inp = synth.small_case(seed, M, N, d=d)
    W, h = inp["W"], inp["h"]
    C, taken = oracle.init(W, d, inp["perm1"], K)
    assert taken == K
    C = C + (0.002 * g.standard_normal(C.shape)).astype(np.float32)
    _, _, _, keep = oracle.select(W, h, oracle.nnz(M, N, p))
    rho = g.uniform(0.5, 2.0, M).astype(np.float32)
    return W, h, C, mask_from_keep(keep, d), rho


def _noalloc(X, hcol, rho, mask, d, C, idx, dist):
    lib = vq.load()
    M, N = X.shape
    st = lib.vq_assign_noalloc(X.data_ptr(), hcol.data_ptr(), rho.data_ptr(), mask.data_ptr(), M, N, d,
                               C.data_ptr(), C.shape[0], idx.data_ptr(), dist.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert st == vq.VQ_OK, lib.vq_last_error().decode()


CASES = [
    (1, 512, 1024, 8, 3000),      # long codebook: block-shared and per-sub-vector searches
    (2, 96, 200, 8, 300),         # smaller input, short codebook
    (3, 257, 520, 8, 2600),       # long again, ragged rows and codebook chunk
]


def test_noalloc_matches_assign_on_consecutive_calls():
    for seed, M, N, d, K in CASES:
        say("noalloc case", (seed, M, N, d, K))
        W, h, C, mask, rho = _case(seed, M, N, d, K)
        Xd, hd, rd, md, Cd = dev(W), dev(h), dev(rho), dev(mask), dev(C)
        ws = vq.workspace(M, N, d, K)
        ref_i, ref_d = vq.assign(Xd, hd, rd, md, d, Cd, ws, want_dist=True)
        n_sub = M * N // d
        for rep in range(2):
            idx = torch.empty(n_sub, dtype=torch.uint16, device="cuda")
            idx.view(torch.int16).fill_(-1)
            dist = torch.full((n_sub,), float("nan"), dtype=torch.float32, device="cuda")
            _noalloc(Xd, hd, rd, md, d, Cd, idx, dist)
            assert bits_equal(host(idx), host(ref_i)), (seed, rep)
            assert bits_equal(host(dist), host(ref_d)), (seed, rep)
        # and the oracle agrees with both
        oi, od = oracle.assign(W, h, rho, keep_from_mask(mask, M, N, d), d, C)
        assert bits_equal(host(ref_i), oi)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    lib = vq.load()
    # 16 M sub-vectors against 65536 centroids need far more than the array holds
    M, N, d, K = 16384, 8192, 8, 65536
    fake = 0x10000
    st = lib.vq_assign_noalloc(fake, fake, None, None, M, N, d, fake, K, fake, None, None)
    assert st == vq.VQ_ERR_INVALID
    assert "scratch" in lib.vq_last_error().decode()
