"""GPU parity of rvq_decode against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import rvq_workloads as W
from gpu_util import needs_gpu, rvq, to_dev, host, announce

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.mark.parametrize("n,q,k", [(1, 1, 1), (37, 8, 1024), (1000, 8, 1024), (513, 32, 1024),
                                   (300, 10, 4096), (99, 3, 65)])
def test_decode_matches_oracle(n, q, k):
    rng = np.random.default_rng(n + q + k)
    books = rng.standard_normal((q, k, 64)).astype(np.float32)
    codes = W.random_codes(n, q, k, seed=n)
    announce("decode", n=n, q=q, k=k)
    out = host(rvq().rvq_decode(to_dev(codes), to_dev(books)))
    np.testing.assert_array_equal(out, oracle.get().decode(codes, books))


def test_decode_order_fixture():
    """Float32 accumulation, stage 0 first: rows 1, 1e8, -1e8 decode to exactly 0."""
    books = np.zeros((3, 1, 64), np.float32)
    books[0, 0, :] = 1.0
    books[1, 0, :] = 1e8
    books[2, 0, :] = -1e8
    codes = np.zeros((5, 3), np.int32)
    out = host(rvq().rvq_decode(to_dev(codes), to_dev(books)))
    assert (out == 0.0).all()


def test_decode_bad_codes_give_nan_rows():
    rng = np.random.default_rng(3)
    books = rng.standard_normal((4, 128, 64)).astype(np.float32)
    codes = W.random_codes(50, 4, 128, seed=4)
    codes[3, 2] = 128
    codes[7, 0] = -1
    codes[9, 3] = 1 << 30
    out = host(rvq().rvq_decode(to_dev(codes), to_dev(books)))
    bad = [3, 7, 9]
    assert np.isnan(out[bad]).all()
    good = np.setdiff1d(np.arange(50), bad)
    np.testing.assert_array_equal(out[good], oracle.get().decode(codes[good], books))


def test_decode_partial_depth_and_leading_dim():
    rng = np.random.default_rng(5)
    books = rng.standard_normal((8, 256, 64)).astype(np.float32)
    codes = W.random_codes(200, 8, 256, seed=6)
    m = rvq()
    out = host(m.rvq_decode(to_dev(codes), to_dev(books), n_stages=3))
    np.testing.assert_array_equal(out, oracle.get().decode(np.ascontiguousarray(codes[:, :3]), books[:3]))


# Codebooks of 4 MiB and more take the stage-ordered kernel: wavefront tiles
# of 32 frames, codes staged 32 stages at a time. Cases cross both.
@pytest.mark.parametrize("n,q,k,ld", [(1, 16, 1024, 16), (31, 33, 1024, 33), (129, 40, 512, 41),
                                      (4099, 64, 256, 64), (700, 8, 4096, 12)])
def test_decode_large_codebook(n, q, k, ld):
    rng = np.random.default_rng(n * 7 + q)
    books = rng.standard_normal((q, k, 64)).astype(np.float32)
    codes = np.full((n, ld), -5, np.int32)   # columns past q are never read
    codes[:, :q] = W.random_codes(n, q, k, seed=n + 1)
    bad = sorted({0, n // 2, n - 1})
    for j, f in enumerate(bad):
        codes[f, (q - 1) if j == 0 else (j * 13) % q] = k if j % 2 == 0 else -1
    announce("decode large codebook", n=n, q=q, k=k, ld=ld)
    out = host(rvq().rvq_decode(to_dev(codes), to_dev(books), n_stages=q))
    assert np.isnan(out[bad]).all()
    good = np.setdiff1d(np.arange(n), bad)
    np.testing.assert_array_equal(out[good], oracle.get().decode(np.ascontiguousarray(codes[good, :q]), books))


@pytest.mark.parametrize("name", ["batched", "deep", "large"])
def test_full_size_decode_sampled(name):
    w = W.WORKLOADS[name]
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    codes = W.random_codes(w.n_frames, w.n_stages, w.n_codes, seed=11)
    announce("decode full size", name=name)
    out = host(rvq().rvq_decode(to_dev(codes), to_dev(books)))
    idx = W.sample_frames(w.n_frames, 8192, seed=12)
    np.testing.assert_array_equal(out[idx], oracle.get().decode(codes[idx], books))
    assert np.isfinite(out).all()
