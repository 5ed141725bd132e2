"""GPU parity of rvq_encode / rvq_roundtrip against the CPU oracle."""

import numpy as np
import pytest

import rvq_workloads as W
from gpu_util import SCORINGS, SPLIT_MAX_FRAMES, needs_gpu, check_encode, widen, rvq, to_dev, host, announce

pytestmark = [pytest.mark.gpu, needs_gpu]


def _books(rng, q, k, d=64, decay=0.5):
    return (rng.standard_normal((q, k, d)) * decay ** np.arange(q)[:, None, None]).astype(np.float32)


@pytest.mark.parametrize("scoring", SCORINGS)
def test_tiny_workload_recovers_construction(scoring):
    w = W.WORKLOADS["tiny"]
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    x, t = W.latents(w, books)
    check_encode(x, books, scoring=scoring)
    m = rvq()
    codes, _ = m.rvq_encode(to_dev(x), to_dev(books))
    np.testing.assert_array_equal(host(codes), t)


@pytest.mark.parametrize("scoring", SCORINGS)
def test_clip_workload_full(scoring):
    w = W.WORKLOADS["clip"]
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    x, _ = W.latents(w, books)
    check_encode(x, books, scoring=scoring)


def _check(x, books, wide, scoring, **kw):
    """check_encode on x itself (split-codebook kernel for small batches) or embedded in a batch
    large enough for the wide kernel."""
    if wide:
        xw, idx = widen(x)
        return check_encode(xw, books, idx=idx, scoring=scoring, **kw)
    return check_encode(x, books, scoring=scoring, **kw)


@pytest.mark.parametrize("n", [1, 31, 129, 677])
@pytest.mark.parametrize("scoring", SCORINGS)
def test_ragged_frame_counts(n, scoring):
    rng = np.random.default_rng(100 + n)
    books = _books(rng, 8, 1024)
    x = rng.standard_normal((n, 64)).astype(np.float32)
    check_encode(x, books, scoring=scoring)


@pytest.mark.parametrize("n", [SPLIT_MAX_FRAMES, SPLIT_MAX_FRAMES + 1, SPLIT_MAX_FRAMES + 31])
@pytest.mark.parametrize("scoring", ["default", "prepared"])
def test_split_threshold_frame_counts(n, scoring):
    """Either side of the split / wide switch, ragged tails included."""
    rng = np.random.default_rng(150 + n)
    books = _books(rng, 4, 1024)
    x = rng.standard_normal((n, 64)).astype(np.float32)
    idx = W.sample_frames(n, 600, seed=n)
    check_encode(x, books, idx=idx, scoring=scoring)


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("k", [1, 63, 64, 65, 100, 1000, 4096])
@pytest.mark.parametrize("scoring", SCORINGS)
def test_codebook_sizes(k, scoring, wide):
    rng = np.random.default_rng(200 + k)
    q = 10 if k == 4096 else 3
    books = _books(rng, q, k)
    x = rng.standard_normal((300, 64)).astype(np.float32)
    _check(x, books, wide, scoring)


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("q,decay", [(1, 1.0), (32, 0.85), (64, 0.9)])
@pytest.mark.parametrize("scoring", SCORINGS)
def test_stage_counts(q, decay, scoring, wide):
    rng = np.random.default_rng(300 + q)
    k = 256 if q == 64 else 1024
    books = _books(rng, q, k, decay=decay)
    x = rng.standard_normal((257, 64)).astype(np.float32)
    _check(x, books, wide, scoring)


def test_partial_depth_prefix():
    """Encoding with the first k of Q stages gives the first k codes (bitrate control)."""
    rng = np.random.default_rng(7)
    books = _books(rng, 8, 1024)
    x = rng.standard_normal((400, 64)).astype(np.float32)
    check_encode(x, books, n_stages=3)
    m = rvq()
    full, _ = m.rvq_encode(to_dev(x), to_dev(books))
    part, _ = m.rvq_encode(to_dev(x), to_dev(books), n_stages=3)
    np.testing.assert_array_equal(host(part), host(full)[:, :3])


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("scoring", SCORINGS)
def test_exact_ties_integer_data(scoring, wide):
    """Small integers: exact scores, many exact ties and duplicated rows (lowest index wins)."""
    rng = np.random.default_rng(8)
    books = rng.integers(-3, 4, size=(4, 128, 64)).astype(np.float32)
    books[:, 100:128] = books[:, 0:28]
    x = rng.integers(-6, 7, size=(500, 64)).astype(np.float32)
    _check(x, books, wide, scoring)


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("scoring", SCORINGS)
def test_all_rows_identical(scoring, wide):
    rng = np.random.default_rng(9)
    books = np.repeat(rng.standard_normal((3, 1, 64)).astype(np.float32), 192, axis=1)
    x = rng.standard_normal((130, 64)).astype(np.float32)
    _check(x, books, wide, scoring)
    codes, _ = rvq().rvq_encode(to_dev(x), to_dev(books))
    assert (host(codes) == 0).all()


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("scoring", SCORINGS)
def test_zero_inputs_and_codebooks(scoring, wide):
    x = np.zeros((70, 64), np.float32)
    books = np.zeros((2, 128, 64), np.float32)
    _check(x, books, wide, scoring)


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("scale", [1e-6, 1e6])
@pytest.mark.parametrize("scoring", SCORINGS)
def test_scaled_data(scale, scoring, wide):
    rng = np.random.default_rng(10)
    books = (_books(rng, 4, 512) * scale).astype(np.float32)
    x = (rng.standard_normal((200, 64)) * scale).astype(np.float32)
    _check(x, books, wide, scoring)


def test_codes_leading_dimension():
    rng = np.random.default_rng(11)
    books = _books(rng, 4, 256)
    x = rng.standard_normal((150, 64)).astype(np.float32)
    import torch
    m = rvq()
    codes = torch.full((150, 7), -5, dtype=torch.int32, device="cuda:0")
    m.rvq_encode(to_dev(x), to_dev(books), codes=codes)
    ref, _ = m.rvq_encode(to_dev(x), to_dev(books))
    c = host(codes)
    np.testing.assert_array_equal(c[:, :4], host(ref))
    assert (c[:, 4:] == -5).all()


def test_deterministic_and_batch_invariant():
    rng = np.random.default_rng(12)
    books = _books(rng, 8, 1024)
    x = rng.standard_normal((1000, 64)).astype(np.float32)
    m = rvq()
    a, ra = m.rvq_encode(to_dev(x), to_dev(books))
    b, rb = m.rvq_encode(to_dev(x), to_dev(books))
    np.testing.assert_array_equal(host(a), host(b))
    np.testing.assert_array_equal(host(ra), host(rb))
    perm = rng.permutation(1000)[:333]
    c, rc = m.rvq_encode(to_dev(x[perm]), to_dev(books))
    np.testing.assert_array_equal(host(c), host(a)[perm])
    np.testing.assert_array_equal(host(rc), host(ra)[perm])


def test_empty_batch_is_noop():
    import torch
    m = rvq()
    books = to_dev(np.zeros((2, 64, 64), np.float32))
    codes, res = m.rvq_encode(torch.empty((0, 64), device="cuda:0"), books)
    assert codes.shape == (0, 2) and res.shape == (0, 64)
    out = m.rvq_decode(torch.empty((0, 2), dtype=torch.int32, device="cuda:0"), books)
    assert out.shape == (0, 64)


@pytest.mark.parametrize("name,count", [("batched", 4096), ("deep", 2048), ("large", 2048)])
@pytest.mark.parametrize("scoring", SCORINGS)
def test_full_size_workloads_sampled(name, count, scoring):
    """Full-size batches in the benchmark's launch configuration; oracle on a seeded sample."""
    w = W.WORKLOADS[name]
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    x, t = W.latents(w, books)
    idx = W.sample_frames(w.n_frames, count, seed=3)
    rep = check_encode(x, books, idx=idx, scoring=scoring)
    announce("full-size report", **rep)
    if w.constructed_from < w.n_frames:
        m = rvq()
        codes, _ = m.rvq_encode(to_dev(x), to_dev(books))
        c = host(codes)[w.constructed_from:]
        frac = (c == t[w.constructed_from:]).all(axis=1).mean()
        announce("constructed recovery", frac=frac)


def test_argument_errors():
    import torch
    m = rvq()
    x = torch.zeros((10, 32), device="cuda:0")
    books = torch.zeros((2, 64, 32), device="cuda:0")
    with pytest.raises(m.RVQError) as e:
        m.rvq_encode(x, books)
    assert e.value.status == m.RVQ_ERR_UNSUPPORTED
    assert m.rvq_encode(torch.zeros((10, 64), device="cuda:0"),
                        torch.zeros((2, 64, 64), device="cuda:0"))[0].shape == (10, 2)


@pytest.mark.parametrize("name", ["batched", "deep", "large"])
def test_scorings_agree_at_full_size(name):
    """Split-bf16 and fp32 scoring give identical codes, residuals and reconstructions."""
    w = W.WORKLOADS[name]
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    x, _ = W.latents(w, books)
    m = rvq()
    xg, bg = to_dev(x), to_dev(books)
    announce("scorings agree", name=name)
    a = [host(t) for t in m.rvq_encode_scored(xg, bg, "bf16x3")]
    b = [host(t) for t in m.rvq_encode_scored(xg, bg, "fp32")]
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_unknown_scoring_rejected():
    m = rvq()
    import torch
    with pytest.raises(ValueError):
        m.rvq_encode_scored(torch.zeros((4, 64), device="cuda:0"), torch.zeros((1, 64, 64), device="cuda:0"), "fp8")


def _bf16_rne(v):
    """float32 -> bfloat16 (round to nearest even) as float32, for finite v."""
    u = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("q,k", [(3, 1000), (2, 256), (1, 1)])
def test_prepared_layout(q, k):
    """rvq_prepare_codebooks: per stage Kp = roundup(K, 256) rows of 8-dim groups (8 hi, 8 lo bf16),
    hi = bf16(v) and lo = bf16(v - hi) round to nearest even; Kp fp32 half-norms (FLT_MAX on padding
    rows, which are zero); the bits of the largest valid half-norm of every 256 rows; stage blocks
    256-byte aligned."""
    m = rvq()
    rng = np.random.default_rng(600 + k)
    books = (rng.standard_normal((q, k, 64)) * 3.0).astype(np.float32)
    books[0, 0] = 0.0
    prep = host(m.rvq_prepare_codebooks(to_dev(books)))
    kp = (k + 255) // 256 * 256
    sbytes = (kp * 260 + 4 * (kp // 256) + 255) // 256 * 256
    assert prep.size >= q * sbytes
    for s in range(q):
        blk = prep[s * sbytes:(s + 1) * sbytes]
        rows = blk[:kp * 256].view(np.uint16).reshape(kp, 8, 2, 8)   # row, group, hi/lo, element
        as_f32 = lambda h: (h.astype(np.uint32) << 16).view(np.float32)
        hi, lo = as_f32(rows[:, :, 0, :]).reshape(kp, 64), as_f32(rows[:, :, 1, :]).reshape(kp, 64)
        want_hi = _bf16_rne(books[s])
        np.testing.assert_array_equal(hi[:k], want_hi)
        np.testing.assert_array_equal(lo[:k], _bf16_rne(books[s] - want_hi))
        assert not rows[k:].any()
        norms = blk[kp * 256:kp * 260].view(np.float32)
        exact = 0.5 * (books[s].astype(np.float64) ** 2).sum(axis=1)
        np.testing.assert_allclose(norms[:k], exact, rtol=1e-6, atol=0)
        assert (norms[k:] == np.finfo(np.float32).max).all()
        maxima = blk[kp * 260:kp * 260 + 4 * (kp // 256)].view(np.uint32)
        for c in range(kp // 256):
            valid = norms[256 * c:min(256 * (c + 1), k)]
            assert maxima[c] == (valid.view(np.uint32).max() if valid.size else 0)
