"""GPU parity of rvq_encode / rvq_roundtrip against the CPU oracle."""

import numpy as np
import pytest

import rvq_workloads as W
from gpu_util import SCORINGS, SPLIT_MAX_FRAMES, PREPARED_SPLIT_MAX_FRAMES, needs_gpu, check_encode, widen, rvq, to_dev, host, announce

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


@pytest.mark.parametrize("n,scoring", [(m, sc) for sc, t in (("default", SPLIT_MAX_FRAMES),
                                                              ("prepared", PREPARED_SPLIT_MAX_FRAMES))
                                        for m in (t, t + 1, t + 31)] + [(SPLIT_MAX_FRAMES, "prepared")])
def test_split_threshold_frame_counts(n, scoring):
    """Either side of the split / wide switch of each path, ragged tails included."""
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
@pytest.mark.parametrize("k", [16384, 20000])
@pytest.mark.parametrize("scoring", SCORINGS)
def test_large_codebooks(k, scoring, wide):
    """Codebooks of many 1024-codeword index spans (16 and 20, the last one partial, K not a multiple
    of 256): the keys' span bookkeeping and the split-codebook kernel's chunk-per-wavefront rotation
    across spans."""
    rng = np.random.default_rng(250 + k)
    books = _books(rng, 2, k)
    x = rng.standard_normal((200, 64)).astype(np.float32)
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


@pytest.mark.parametrize("q,k", [(8, 1024), (5, 300), (3, 4096)])
def test_prepared_batch_invariant_across_kernels(q, k):
    """The same frames encoded from prepared codebooks inside a batch that takes the wide kernel and
    alone as batches that take the split-codebook kernel (8,192 frames, its largest, and 333) give the
    same codes, residuals and reconstructions, all frames compared (both kernels decide every stage
    exactly, so neither may differ from the other in any frame)."""
    rng = np.random.default_rng(40 + k)
    books = _books(rng, q, k)
    x = rng.standard_normal((20000, 64)).astype(np.float32)
    x[10000:] = (x[10000:] * 1e-3).astype(np.float32)   # small residuals too
    m = rvq()
    bg = to_dev(books)
    prep = m.rvq_prepare_codebooks(bg)
    announce("prepared batch invariance", n=20000, q=q, k=k)
    wc, wr, wres = (host(t) for t in m.rvq_encode_prepared(to_dev(x), bg, prep, recon=True))
    perm = rng.permutation(20000)
    for sub in (perm[:8192], perm[8192:8192 + 333]):
        announce("prepared batch invariance, split kernel", n=sub.size, q=q, k=k)
        c, r, res = (host(t) for t in m.rvq_encode_prepared(to_dev(x[sub]), bg, prep, recon=True))
        np.testing.assert_array_equal(c, wc[sub])
        np.testing.assert_array_equal(res, wres[sub])
        np.testing.assert_array_equal(r, wr[sub])


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


def _stage_layout(k):
    """(Kp, stage block bytes) of the prepared layout."""
    kp = (k + 255) // 256 * 256
    return kp, (kp * 144 + 4 * (kp // 256) + 4 + 255) // 256 * 256


def _stage_exp(book):
    """Power-of-two scale e of a stage: max |c| * 2^e in [1/2, 1), clamped to [-15, 24]."""
    amax = float(np.abs(book).max())
    return 0 if amax == 0.0 else int(np.clip(-np.frexp(amax)[1], -15, 24))


@pytest.mark.parametrize("q,k", [(3, 1000), (2, 256), (1, 1)])
def test_prepared_layout(q, k):
    """rvq_prepare_codebooks: per stage Kp = roundup(K, 256) rows of 144 bytes, fp16 (round to
    nearest even) of c' = 2^e c with the stage's power of two e, then the two fp16 parts of
    0.5*||c'||^2 and zeros (padding rows all zero); the largest of those per 256 rows; e. Stage
    blocks 256-byte aligned."""
    m = rvq()
    rng = np.random.default_rng(600 + k)
    books = (rng.standard_normal((q, k, 64)) * 3.0 * 4.0 ** -np.arange(q)[:, None, None]).astype(np.float32)
    books[0, 0] = 0.0
    prep = host(m.rvq_prepare_codebooks(to_dev(books)))
    kp, sbytes = _stage_layout(k)
    assert prep.size >= q * sbytes
    for s in range(q):
        blk = prep[s * sbytes:(s + 1) * sbytes]
        e = _stage_exp(books[s])
        assert blk[kp * 144 + 4 * (kp // 256):][:4].view(np.int32)[0] == e
        scaled = (books[s].astype(np.float64) * 2.0 ** e).astype(np.float32)   # exact: a power of two
        rows = blk[:kp * 144].view(np.uint16).reshape(kp, 72)
        rows16 = rows[:, :64]
        np.testing.assert_array_equal(rows16[:k], scaled.astype(np.float16).view(np.uint16))
        assert not rows16[k:].any()
        assert not rows[:, 66:].any()   # zeros after the half-norm parts
        parts = rows[:, 64:66].copy().view(np.float16).astype(np.float64)
        want = 0.5 * (scaled.astype(np.float64) ** 2).sum(axis=1)
        got = parts[:k, 0] + parts[:k, 1]
        assert (np.abs(got - want) <= 2e-6 * want + 2.0 ** -24).all()
        # the high part is the fp16 rounding of the sum of both parts
        np.testing.assert_array_equal(parts[:k, 0], got.astype(np.float16).astype(np.float64))
        assert not parts[k:].any()
        max16 = blk[kp * 144:kp * 144 + 4 * (kp // 256)].view(np.float32)
        for c in range(kp // 256):
            w = want[256 * c:min(256 * (c + 1), k)]
            assert max16[c] == pytest.approx(w.max() if w.size else 0.0, rel=2e-6, abs=1e-30)


def test_prepared_out_of_fp16_range():
    """A stage with entries beyond 2^20 is marked by infinite maxima; an all-zero stage has e = 0."""
    m = rvq()
    rng = np.random.default_rng(610)
    books = rng.standard_normal((3, 300, 64)).astype(np.float32)
    books[1] *= 2.0 ** 22
    books[2] = 0.0
    prep = host(m.rvq_prepare_codebooks(to_dev(books)))
    kp, sbytes = _stage_layout(300)
    for s, inf in ((0, False), (1, True), (2, False)):
        blk = prep[s * sbytes:(s + 1) * sbytes]
        max16 = blk[kp * 144:kp * 144 + 4 * (kp // 256)].view(np.float32)
        assert bool(np.isinf(max16).all()) == inf and bool(np.isinf(max16).any()) == inf
        assert blk[kp * 144 + 4 * (kp // 256):][:4].view(np.int32)[0] == _stage_exp(books[s])


@pytest.mark.parametrize("case", ["huge_stage", "huge_residual", "some_huge_residuals", "tiny_residual",
                                  "near_duplicates", "clustered"])
@pytest.mark.parametrize("wide", [False, True])
def test_prepared_fp16_edges(case, wide):
    """Small and wide batches through the prepared path: a stage out of the fp16 range, residuals out of it
    (both resolved by the float64 rescan; for some frames of each wavefront only, the others decided
    as usual), residuals in the fp16 subnormal range, near-duplicate
    rows (re-rank within one key set) and rows clustered so tightly that frames hold many
    candidates."""
    rng = np.random.default_rng(620)
    books = _books(rng, 4, 1024)
    x = rng.standard_normal((400, 64)).astype(np.float32)
    if case == "huge_stage":
        books[1] *= 2.0 ** 22
    elif case == "huge_residual":
        x *= 1e5
    elif case == "some_huge_residuals":   # every third frame out of fp16's range, the rest not
        x[::3] *= 1e5
    elif case == "tiny_residual":
        books *= 1e-6
        x *= 1e-6
    elif case == "near_duplicates":
        books[:, 1::2] = books[:, 0::2] * (1.0 + 1e-5 * rng.standard_normal((4, 512, 64))).astype(np.float32)
    else:
        centre = rng.standard_normal((4, 1, 64)).astype(np.float32)
        books = (centre + 1e-3 * rng.standard_normal((4, 1024, 64))).astype(np.float32)
        x = (centre[0] + 1e-3 * rng.standard_normal((400, 64))).astype(np.float32)
    _check(x, books, wide, "prepared")


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("seed", range(6))
def test_prepared_random_shapes_and_scales(seed, wide):
    """fp16-scored paths (small and wide batches) under random stage counts, codebook sizes (not multiples of 64), per-stage
    codebook scales from 1e-3 to 1e3 (stage exponents across their range), residual scales, and
    near-duplicate rows; codes, residuals and reconstructions against the oracle."""
    rng = np.random.default_rng(700 + seed)
    q = int(rng.integers(1, 6))
    k = int(rng.integers(1, 1100))
    scales = 10.0 ** rng.uniform(-3, 3, size=q)
    books = (rng.standard_normal((q, k, 64)) * scales[:, None, None]).astype(np.float32)
    if seed % 2 == 1 and k > 8:   # near-duplicate rows in every stage
        j = rng.integers(0, k, size=k // 4)
        books[:, j] = books[:, rng.integers(0, k, size=j.size)] * (
            1.0 + 1e-6 * rng.standard_normal((q, j.size, 64))).astype(np.float32)
    x = (rng.standard_normal((300, 64)) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
    _check(x, books, wide, "prepared")


@pytest.mark.parametrize("case", ["mixed_dims", "subnormal_frames", "clamped_scale_stage", "zero_frames_and_rows",
                                  "sparse_integer"])
@pytest.mark.parametrize("wide", [False, True])
def test_prepared_value_extremes(case, wide):
    """Small and wide batches through the fp16-scored paths on value patterns the random cases do not reach:
    per-dimension scales spread over eight decades (the bound's norm terms dominated by a few
    dimensions), frames of float32 subnormals (flushed by the fp16 conversion, decided by the
    bound's absolute terms), a stage whose scale exponent is clamped (entries near 1e-12, fp16
    subnormal after scaling), all-zero frames against duplicated all-zero codewords (equal scores,
    lowest index), and sparse integer data with exact ties at K not a multiple of 64."""
    rng = np.random.default_rng(800)
    k = 1000
    books = _books(rng, 4, k)
    x = rng.standard_normal((400, 64)).astype(np.float32)
    if case == "mixed_dims":
        dim_scale = (10.0 ** rng.uniform(-4, 4, size=64)).astype(np.float32)
        books = (books * dim_scale).astype(np.float32)
        x = (x * dim_scale).astype(np.float32)
    elif case == "subnormal_frames":
        x[::3] = (x[::3] * 1e-39).astype(np.float32)
        assert np.all(np.abs(x[::3]) < np.finfo(np.float32).tiny)
    elif case == "clamped_scale_stage":
        books[2] = (books[2] * 1e-12).astype(np.float32)
    elif case == "zero_frames_and_rows":
        x[::4] = 0.0
        books[:, [5, 77, 600, 601, 999]] = 0.0
    else:
        books = (rng.integers(-2, 3, size=(4, k, 64)) * (rng.random((4, k, 64)) < 0.1)).astype(np.float32)
        x = (rng.integers(-3, 4, size=(400, 64)) * (rng.random((400, 64)) < 0.2)).astype(np.float32)
    _check(x, books, wide, "prepared")


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("k", [1, 65, 100, 1000, 1024])
@pytest.mark.parametrize("scoring", SCORINGS)
def test_out_of_range_and_nonfinite_frames(k, scoring, wide):
    """Every third frame holds entries beyond fp16's 65504 (the fp16-scored path decides those by the
    float64 rescan at every stage, the last included) and shares its wavefronts with ordinary frames
    that need a re-rank (near-duplicate rows); one frame holds a NaN and one an infinity. Codes
    decoded from such frames' keys may name padding slots past K; they must never be used as row
    indices. Finite frames equal the oracle bit for bit; every code lies in [0, K)."""
    rng = np.random.default_rng(900 + k)
    books = _books(rng, 4, k)
    if k > 1:
        half = k // 2
        books[:, half:2 * half] = books[:, :half] * (
            1.0 + 1e-5 * rng.standard_normal((4, half, 64))).astype(np.float32)
    x = rng.standard_normal((400, 64)).astype(np.float32)
    x[::3] *= 1e5
    x[5, 10] = np.nan
    x[7, 3] = np.inf
    nonfinite = np.nonzero(~np.isfinite(x).all(axis=1))[0]
    xw, idx = widen(x) if wide else (x, np.arange(x.shape[0]))
    sel = np.setdiff1d(idx, nonfinite)
    check_encode(xw, books, idx=sel, scoring=scoring)
    m = rvq()
    xg, bg = to_dev(xw), to_dev(books)
    if scoring == "default":
        codes, _ = m.rvq_encode(xg, bg)
    elif scoring == "prepared":
        codes, _, _ = m.rvq_encode_prepared(xg, bg, m.rvq_prepare_codebooks(bg))
    else:
        codes, _, _ = m.rvq_encode_scored(xg, bg, scoring)
    c = host(codes)
    assert c.min() >= 0 and c.max() < k


def test_shape_mismatches_rejected():
    """The C ABI takes the latent width from x alone, and the code rows from n_frames: the binding
    rejects codebooks of another width and output codes of the wrong shape before any launch."""
    import torch
    m = rvq()
    dev = "cuda:0"
    x = torch.zeros((10, 64), device=dev)
    narrow = torch.zeros((2, 64, 8), device=dev)
    books = torch.zeros((2, 64, 64), device=dev)
    prep = m.rvq_prepare_codebooks(books)
    for call in (lambda: m.rvq_encode(x, narrow), lambda: m.rvq_roundtrip(x, narrow),
                 lambda: m.rvq_encode_scored(x, narrow, "fp32"),
                 lambda: m.rvq_encode_prepared(x, narrow, prep)):
        with pytest.raises(ValueError):
            call()
    short = torch.zeros((9, 2), dtype=torch.int32, device=dev)
    thin = torch.zeros((10, 1), dtype=torch.int32, device=dev)
    for codes in (short, thin):
        with pytest.raises(ValueError):
            m.rvq_encode(x, books, codes=codes)
        with pytest.raises(ValueError):
            m.rvq_encode_scored(x, books, "fp32", out=(codes, None, None))
        with pytest.raises(ValueError):
            m.rvq_encode_prepared(x, books, prep, out=(codes, None, None))
