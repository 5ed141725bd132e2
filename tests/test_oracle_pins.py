"""The CPU oracle against its pins (no GPU)."""

import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_workload_tiny_recovers_construction(oracle_lib):
    """The tiny round trip's frames are sums of codewords plus sigma=1e-3 noise: codes == t."""
    import numpy as np
    import rvq_workloads as W
    w = W.WORKLOADS["tiny"]
    cb = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    x, t = W.latents(w, cb)
    codes, residual, best, second = oracle_lib.encode(x, cb)
    np.testing.assert_array_equal(codes, t)
    recon = oracle_lib.decode(codes, cb)
    assert np.abs(recon + residual - x).max() < 1e-5


def test_threads_do_not_change_results(oracle_lib):
    """Parallel over frame ranges == serial (frames are independent)."""
    import numpy as np
    rng = np.random.default_rng(5)
    x = rng.standard_normal((97, 16)).astype(np.float32)
    cb = rng.standard_normal((3, 64, 16)).astype(np.float32)
    a = oracle_lib.encode(x, cb, threads=1)
    b = oracle_lib.encode(x, cb, threads=7)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
