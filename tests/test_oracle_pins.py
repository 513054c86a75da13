"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle as O
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def test_oracle_wrapper_keeps_converted_inputs_alive(orc):
    """Inputs the wrapper must convert (float64, Fortran order, strided views) give
    the same results as contiguous float32 ones: the converted copies stay alive
    for the whole C call."""
    g = np.random.default_rng(5)
    M, N, d, K = 12, 16, 4, 6
    C = g.standard_normal((K, d)).astype(np.float32)
    idx = g.integers(0, K, M * N // d).astype(np.uint16)
    c = g.uniform(0.5, 2.0, N).astype(np.float32)
    ref = O.reconstruct(M, N, d, C, idx, c=c, lib=orc)
    big = np.zeros((K, 2 * d), np.float64)
    big[:, ::2] = C
    got = O.reconstruct(M, N, d, np.asfortranarray(C.astype(np.float64)), idx.astype(np.int64),
                        c=c.astype(np.float64), lib=orc)
    got2 = O.reconstruct(M, N, d, big[:, ::2], idx, c=c, lib=orc)
    assert np.array_equal(got, ref) and np.array_equal(got2, ref)
