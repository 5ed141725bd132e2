"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises
``AssertionError`` on a mismatch. ``test_oracle_pins.py`` runs them on the
real oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle
with planted mistakes and expects every copy to fail at least one.

What pins what:

* hand-worked example (tests/golden/encode_handworked.txt): codes, both
  distances, residual and reconstruction of a 3-stage, 4-codeword, 2-dim
  case with exact ties -- pins the distance, the tie rule, the stage order
  and the sign of the residual update;
* decode order (tests/golden/decode_order.txt): float32 accumulation with
  stage 0 first;
* one stage against scipy's ``cdist`` 1-nearest-neighbour (library routine);
* every stage against ``cdist`` on the residual that a shorter encode
  returns (so the residual chain is pinned stage by stage);
* exact recovery of codes from inputs built as sums of well-separated
  codewords (closed form), with the residual norm non-increasing;
* the identity "smallest distance of a stage equals the squared norm of
  the residual that stage leaves";
* exact integer arithmetic with duplicated rows (lowest index on ties,
  recon + residual == x exactly);
* invariants: prefix consistency, frame permutation, decode of one stage is
  a row gather, out-of-range codes give a NaN frame;
* linear layer against numpy's float64 matmul;
* per-stage projected encode / decode: a hand-worked 2-stage case with a
  three-way tie (tests/golden/projected_handworked.txt); identity
  projections reduce it to the plain encode / decode; small-integer data
  against an exact integer re-derivation with numpy (argmin first
  occurrence); the argmin follows given encodings (checked with cdist);
  prefix consistency; the float32, stage-0-first decode order; NaN frames
  for bad codes;
* normalized (cosine) variant: a hand-worked 2-stage case where the
  normalization decides a pick (tests/golden/cosine_handworked.txt); the
  argmin equals scipy's cosine-distance argmin; scaling an encoding or a
  codeword by a positive factor changes nothing; the zero encoding and a
  zero codeword follow the 1e-12 norm floor.
"""

import numpy as np
from scipy.spatial.distance import cdist

import golden_io


def pin_handworked(o):
    books, frames = golden_io.read("encode_handworked.txt")
    x = np.array([f["x"] for f in frames], np.float32)
    codes, residual, best, second = o.encode(x, books)
    np.testing.assert_array_equal(codes, np.array([f["codes"] for f in frames], np.int32))
    np.testing.assert_array_equal(best, np.array([f["best"] for f in frames]))
    np.testing.assert_array_equal(second, np.array([f["second"] for f in frames]))
    np.testing.assert_array_equal(residual, np.array([f["residual"] for f in frames], np.float32))
    recon = o.decode(codes, books)
    np.testing.assert_array_equal(recon, np.array([f["recon"] for f in frames], np.float32))


def pin_decode_order(o):
    books, frames = golden_io.read("decode_order.txt")
    codes = np.array([f["codes"] for f in frames], np.int32)
    recon = o.decode(codes, books)
    np.testing.assert_array_equal(recon, np.array([f["recon"] for f in frames], np.float32))


def _random_books(rng, q, k, d, decay=0.5):
    return (rng.standard_normal((q, k, d)) * decay ** np.arange(q)[:, None, None]).astype(np.float32)


def _check_nn(codes_q, dist, what):
    """codes_q must be the first-occurrence argmin of dist, up to float64 rounding of cdist."""
    ref = np.argmin(dist, axis=1)
    rows = np.arange(dist.shape[0])
    bad = codes_q != ref
    if bad.any():
        a, b = dist[rows[bad], codes_q[bad]], dist[rows[bad], ref[bad]]
        assert np.all(np.abs(a - b) <= 1e-12 * np.abs(b)), f"{what}: picks differ from cdist argmin"


def pin_single_stage_cdist(o):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((300, 7)).astype(np.float32)
    books = _random_books(rng, 1, 257, 7)
    codes, residual, best, second = o.encode(x, books)
    dist = cdist(x.astype(np.float64), books[0].astype(np.float64), "sqeuclidean")
    _check_nn(codes[:, 0], dist, "stage 0")
    srt = np.sort(dist, axis=1)
    np.testing.assert_allclose(best[:, 0], srt[:, 0], rtol=1e-12, atol=0)
    np.testing.assert_allclose(second[:, 0], srt[:, 1], rtol=1e-12, atol=0)
    np.testing.assert_array_equal(residual, x - books[0][codes[:, 0]])


def pin_every_stage_cdist(o):
    rng = np.random.default_rng(12)
    q, k, d = 4, 96, 9
    x = rng.standard_normal((200, d)).astype(np.float32)
    books = _random_books(rng, q, k, d)
    codes, _, best, _ = o.encode(x, books)
    r = x
    for s in range(q):
        dist = cdist(r.astype(np.float64), books[s].astype(np.float64), "sqeuclidean")
        _check_nn(codes[:, s], dist, f"stage {s}")
        np.testing.assert_allclose(best[:, s], dist.min(axis=1), rtol=1e-12, atol=0)
        # the residual entering stage s+1 is what an (s+1)-stage encode leaves
        _, r, _, _ = o.encode(x, books, n_stages=s + 1)


def pin_constructed_recovery(o):
    rng = np.random.default_rng(13)
    q, k, d, n = 8, 1024, 64, 400
    books = _random_books(rng, q, k, d)
    t = rng.integers(0, k, size=(n, q))
    exact = np.zeros((n, d))
    for s in range(q):
        exact += books[s][t[:, s]].astype(np.float64)
    x = (exact + 1e-3 * rng.standard_normal((n, d))).astype(np.float32)
    codes, residual, best, _ = o.encode(x, books)
    np.testing.assert_array_equal(codes, t.astype(np.int32))
    np.testing.assert_allclose(residual, x.astype(np.float64) - exact, rtol=0, atol=1e-5)
    # ||r_{s+1}||^2 equals stage s's best distance: non-increasing on these inputs
    norms = np.concatenate([np.sum(x.astype(np.float64) ** 2, axis=1)[:, None], best], axis=1)
    assert np.all(np.diff(norms, axis=1) <= 1e-9 * norms[:, :-1]), "residual norm grew"


def pin_best_is_residual_norm(o):
    rng = np.random.default_rng(14)
    q, k, d = 5, 128, 16
    x = rng.standard_normal((250, d)).astype(np.float32)
    books = _random_books(rng, q, k, d, decay=0.7)
    _, _, best, _ = o.encode(x, books)
    for s in range(q):
        _, r, _, _ = o.encode(x, books, n_stages=s + 1)
        rn = np.sum(r.astype(np.float64) ** 2, axis=1)
        np.testing.assert_allclose(best[:, s], rn, rtol=1e-6, atol=1e-12)


def pin_integer_exact(o):
    rng = np.random.default_rng(15)
    q, k, d, n = 4, 64, 16, 300
    books = rng.integers(-4, 5, size=(q, k, d)).astype(np.float32)
    books[:, 40:48] = books[:, 8:16]        # duplicated rows: lower copy must win
    x = rng.integers(-8, 9, size=(n, d)).astype(np.float32)
    codes, residual, best, second = o.encode(x, books)
    dup = (codes >= 40) & (codes < 48)
    assert not dup.any(), "a duplicated row won over its lower-index copy"
    recon = o.decode(codes, books)
    np.testing.assert_array_equal(recon + residual, x)
    gathered = np.stack([books[s][codes[:, s]] for s in range(q)], axis=1)
    np.testing.assert_array_equal(recon, gathered.sum(axis=1))
    # integer distances are exact: every pick is the first minimum
    r = x.astype(np.int64)
    for s in range(q):
        dist = ((r[:, None, :] - books[s].astype(np.int64)[None]) ** 2).sum(axis=2)
        np.testing.assert_array_equal(codes[:, s], np.argmin(dist, axis=1))
        np.testing.assert_array_equal(best[:, s], dist.min(axis=1).astype(np.float64))
        np.testing.assert_array_equal(second[:, s], np.sort(dist, axis=1)[:, 1].astype(np.float64))
        r = r - books[s].astype(np.int64)[codes[:, s]]


def pin_prefix_and_permutation(o):
    rng = np.random.default_rng(16)
    q, k, d, n = 6, 128, 12, 180
    x = rng.standard_normal((n, d)).astype(np.float32)
    books = _random_books(rng, q, k, d)
    codes, residual, best, second = o.encode(x, books)
    c3, _, b3, s3 = o.encode(x, books, n_stages=3)
    np.testing.assert_array_equal(c3, codes[:, :3])
    np.testing.assert_array_equal(b3, best[:, :3])
    np.testing.assert_array_equal(s3, second[:, :3])
    perm = rng.permutation(n)
    cp, rp, _, _ = o.encode(x[perm], books)
    np.testing.assert_array_equal(cp, codes[perm])
    np.testing.assert_array_equal(rp, residual[perm])


def pin_decode_gather(o):
    rng = np.random.default_rng(17)
    books = _random_books(rng, 3, 50, 10)
    codes = rng.integers(0, 50, size=(64, 1)).astype(np.int32)
    np.testing.assert_array_equal(o.decode(codes, books[:1]), books[0][codes[:, 0]])
    codes3 = rng.integers(0, 50, size=(64, 3)).astype(np.int32)
    codes3[5, 1] = 50
    codes3[9, 2] = -1
    out = o.decode(codes3, books)
    assert np.isnan(out[5]).all() and np.isnan(out[9]).all()
    ok = np.ones(64, bool)
    ok[[5, 9]] = False
    assert np.isfinite(out[ok]).all()
    # exact when the rows are small integers (any summation order agrees)
    ib = rng.integers(-100, 100, size=(3, 50, 10)).astype(np.float32)
    codes3 = rng.integers(0, 50, size=(64, 3)).astype(np.int32)
    ref = sum(ib[s][codes3[:, s]] for s in range(3))
    np.testing.assert_array_equal(o.decode(codes3, ib), ref)


def pin_linear(o):
    rng = np.random.default_rng(18)
    h = rng.standard_normal((37, 1024)).astype(np.float32)
    w = rng.standard_normal((5, 1024)).astype(np.float32)
    b = rng.standard_normal(5).astype(np.float32)
    y = o.linear(h, w, b)
    # a float64 sum rounded once agrees with numpy's float64 matmul rounded once
    # (they differ only within ~1e-16 of a float32 rounding boundary)
    ref = h.astype(np.float64) @ w.astype(np.float64).T + b.astype(np.float64)
    np.testing.assert_array_equal(y, ref.astype(np.float32))
    y0 = o.linear(h, w, None)
    np.testing.assert_array_equal(y0, (h.astype(np.float64) @ w.astype(np.float64).T).astype(np.float32))
    hi = rng.integers(-3, 4, size=(9, 6)).astype(np.float32)
    wi = rng.integers(-3, 4, size=(4, 6)).astype(np.float32)
    np.testing.assert_array_equal(o.linear(hi, wi), hi @ wi.T)


def _projected_case(name):
    p, frames = golden_io.read_projected(name)
    h = np.array([f["h"] for f in frames], np.float32)
    return p, frames, h


def pin_projected_handworked(o):
    p, frames, h = _projected_case("projected_handworked.txt")
    q, _, d = p["books"].shape
    codes, e, residual, best, second = o.projected_encode(h, p["w_in"], p["b_in"], p["books"],
                                                          p["w_out"], p["b_out"])
    np.testing.assert_array_equal(codes, np.array([f["codes"] for f in frames], np.int32))
    np.testing.assert_array_equal(e.transpose(1, 0, 2).reshape(len(frames), q * d),
                                  np.array([f["e"] for f in frames], np.float32))
    np.testing.assert_array_equal(best, np.array([f["best"] for f in frames]))
    np.testing.assert_array_equal(second, np.array([f["second"] for f in frames]))
    np.testing.assert_array_equal(residual, np.array([f["residual"] for f in frames], np.float32))
    recon = o.projected_decode(codes, p["books"], p["w_out"], p["b_out"])
    np.testing.assert_array_equal(recon, np.array([f["recon"] for f in frames], np.float32))


def pin_projected_identity_is_plain_rvq(o):
    rng = np.random.default_rng(21)
    q, k, d, n = 4, 96, 16, 150
    x = rng.standard_normal((n, d)).astype(np.float32)
    books = _random_books(rng, q, k, d)
    eye = np.broadcast_to(np.eye(d, dtype=np.float32), (q, d, d))
    zeros_in, zeros_out = np.zeros((q, d), np.float32), np.zeros((q, d), np.float32)
    codes, e, residual, best, second = o.projected_encode(x, eye, zeros_in, books, eye, zeros_out)
    c0, r0, b0, s0 = o.encode(x, books)
    np.testing.assert_array_equal(codes, c0)
    np.testing.assert_array_equal(residual, r0)
    np.testing.assert_array_equal(best, b0)
    np.testing.assert_array_equal(second, s0)
    np.testing.assert_array_equal(e[0], x)
    for s in range(1, q):
        _, rs, _, _ = o.encode(x, books, n_stages=s)
        np.testing.assert_array_equal(e[s], rs)
    np.testing.assert_array_equal(o.projected_decode(codes, books, eye, None), o.decode(codes, books))


def pin_projected_integer_exact(o):
    rng = np.random.default_rng(22)
    q, k, d, hid, n = 3, 12, 3, 7, 400
    books = rng.integers(-3, 4, size=(q, k, d)).astype(np.float32)
    books[:, 9:12] = books[:, 2:5]          # duplicated rows: lower copy must win
    w_in = rng.integers(-2, 3, size=(q, d, hid)).astype(np.float32)
    b_in = rng.integers(-2, 3, size=(q, d)).astype(np.float32)
    w_out = rng.integers(-2, 3, size=(q, hid, d)).astype(np.float32)
    b_out = rng.integers(-2, 3, size=(q, hid)).astype(np.float32)
    h = rng.integers(-5, 6, size=(n, hid)).astype(np.float32)
    codes, e, residual, best, second = o.projected_encode(h, w_in, b_in, books, w_out, b_out)
    r = h.astype(np.int64)
    recon = np.zeros((n, hid), np.int64)
    for s in range(q):
        es = r @ w_in[s].astype(np.int64).T + b_in[s].astype(np.int64)
        np.testing.assert_array_equal(e[s], es.astype(np.float32))
        dist = ((es[:, None, :] - books[s].astype(np.int64)[None]) ** 2).sum(axis=2)
        np.testing.assert_array_equal(codes[:, s], np.argmin(dist, axis=1))
        np.testing.assert_array_equal(best[:, s], dist.min(axis=1).astype(np.float64))
        np.testing.assert_array_equal(second[:, s], np.sort(dist, axis=1)[:, 1].astype(np.float64))
        ps = books[s].astype(np.int64)[codes[:, s]] @ w_out[s].astype(np.int64).T + b_out[s].astype(np.int64)
        r = r - ps
        recon = recon + ps
    np.testing.assert_array_equal(residual, r.astype(np.float32))
    out = o.projected_decode(codes, books, w_out, b_out)
    np.testing.assert_array_equal(out, recon.astype(np.float32))
    np.testing.assert_array_equal(out + residual, h)


def pin_projected_follows_given_encodings(o):
    rng = np.random.default_rng(23)
    q, k, d, hid, n = 3, 64, 8, 48, 200
    books = _random_books(rng, q, k, d)
    w_in = (rng.standard_normal((q, d, hid)) / np.sqrt(hid)).astype(np.float32)
    w_out = (rng.standard_normal((q, hid, d)) / np.sqrt(d)).astype(np.float32)
    b_in = (0.1 * rng.standard_normal((q, d))).astype(np.float32)
    b_out = (0.1 * rng.standard_normal((q, hid))).astype(np.float32)
    h = rng.standard_normal((n, hid)).astype(np.float32)
    given = rng.standard_normal((q, n, d)).astype(np.float32)
    codes, e, residual, best, _ = o.projected_encode(h, w_in, b_in, books, w_out, b_out, e_given=given)
    r = h.astype(np.float64)
    for s in range(q):
        dist = cdist(given[s].astype(np.float64), books[s].astype(np.float64), "sqeuclidean")
        _check_nn(codes[:, s], dist, f"stage {s}")
        np.testing.assert_allclose(best[:, s], dist.min(axis=1), rtol=1e-12, atol=0)
        # the oracle's own projection is taken on the residual that the given picks leave
        np.testing.assert_allclose(e[s], r @ w_in[s].astype(np.float64).T + b_in[s], rtol=0, atol=1e-5)
        r = r - (books[s][codes[:, s]].astype(np.float64) @ w_out[s].astype(np.float64).T + b_out[s])
    np.testing.assert_allclose(residual, r, rtol=0, atol=1e-5)
    # without given encodings the picks are made on the oracle's own projections
    c_own, e_own, _, _, _ = o.projected_encode(h, w_in, b_in, books, w_out, b_out)
    c_again, _, _, _, _ = o.projected_encode(h, w_in, b_in, books, w_out, b_out, e_given=e_own)
    np.testing.assert_array_equal(c_again, c_own)
    assert (c_own != codes).any(), "random given encodings should change some picks"


def pin_projected_prefix_and_decode(o):
    rng = np.random.default_rng(24)
    q, k, d, hid, n = 5, 64, 8, 32, 120
    books = _random_books(rng, q, k, d)
    w_in = (rng.standard_normal((q, d, hid)) / np.sqrt(hid)).astype(np.float32)
    w_out = (rng.standard_normal((q, hid, d)) / np.sqrt(d)).astype(np.float32)
    h = rng.standard_normal((n, hid)).astype(np.float32)
    codes, e, _, best, _ = o.projected_encode(h, w_in, None, books, w_out, None)
    c2, e2, _, b2, _ = o.projected_encode(h, w_in, None, books, w_out, None, n_stages=2)
    np.testing.assert_array_equal(c2, codes[:, :2])
    np.testing.assert_array_equal(e2, e[:2])
    np.testing.assert_array_equal(b2, best[:, :2])
    # decode: float32 accumulation, stage 0 first (rows 1, 1e8, -1e8 give 0)
    books3 = np.zeros((3, 1, 1), np.float32)
    books3[:, 0, 0] = (1.0, 1e8, -1e8)
    one = np.ones((3, 1, 1), np.float32)
    out = o.projected_decode(np.zeros((4, 3), np.int32), books3, one, None)
    assert (out == 0.0).all()
    bad = codes.copy()
    bad[3, 1] = k
    bad[7, 4] = -1
    out = o.projected_decode(bad, books, w_out, None)
    assert np.isnan(out[[3, 7]]).all() and np.isfinite(np.delete(out, [3, 7], axis=0)).all()


def pin_cosine_handworked(o):
    p, frames, h = _projected_case("cosine_handworked.txt")
    q, _, d = p["books"].shape
    codes, e, residual, best, second = o.projected_encode(h, p["w_in"], p["b_in"], p["books"],
                                                          p["w_out"], p["b_out"], normalize=True)
    np.testing.assert_array_equal(codes, np.array([f["codes"] for f in frames], np.int32))
    np.testing.assert_array_equal(e.transpose(1, 0, 2).reshape(len(frames), q * d),
                                  np.array([f["e"] for f in frames], np.float32))
    np.testing.assert_allclose(best, np.array([f["best"] for f in frames]), rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(second, np.array([f["second"] for f in frames]), rtol=1e-9, atol=1e-15)
    np.testing.assert_array_equal(residual, np.array([f["residual"] for f in frames], np.float32))
    recon = o.projected_decode(codes, p["books"], p["w_out"], p["b_out"])
    np.testing.assert_array_equal(recon, np.array([f["recon"] for f in frames], np.float32))


def pin_cosine_against_cdist(o):
    rng = np.random.default_rng(25)
    q, k, d, hid, n = 3, 200, 8, 40, 300
    books = rng.standard_normal((q, k, d)).astype(np.float32)
    w_in = (rng.standard_normal((q, d, hid)) / np.sqrt(hid)).astype(np.float32)
    w_out = (rng.standard_normal((q, hid, d)) / np.sqrt(d)).astype(np.float32)
    b_in = (0.05 * rng.standard_normal((q, d))).astype(np.float32)
    h = rng.standard_normal((n, hid)).astype(np.float32)
    codes, e, _, best, _ = o.projected_encode(h, w_in, b_in, books, w_out, None, normalize=True)
    for s in range(q):
        cosd = cdist(e[s].astype(np.float64), books[s].astype(np.float64), "cosine")   # 1 - cos
        _check_nn(codes[:, s], cosd, f"stage {s}")
        np.testing.assert_allclose(best[:, s], 2.0 * cosd.min(axis=1), rtol=1e-9, atol=1e-12)
    # a positive scale of an encoding or of a codeword changes no pick
    scaled = books * rng.uniform(0.1, 10.0, size=(q, k, 1)).astype(np.float32)
    given = e * rng.uniform(0.1, 10.0, size=(q, n, 1)).astype(np.float32)
    c2, _, _, _, _ = o.projected_encode(h, w_in, b_in, scaled, w_out, None, e_given=given, normalize=True)
    np.testing.assert_array_equal(c2[:, 0], codes[:, 0])
    # without normalization the picks differ on these codebooks
    c_plain, _, _, _, _ = o.projected_encode(h, w_in, b_in, books, w_out, None)
    assert (c_plain[:, 0] != codes[:, 0]).any()


def pin_cosine_norm_floor(o):
    # codewords (2,0), (0,3), (0,0): a zero encoding stays zero, so every distance is |v_k|^2 =
    # 1, 1, 0 and the zero codeword wins; a nonzero encoding is at distance 1 from the zero codeword
    books = np.array([[[2.0, 0.0], [0.0, 3.0], [0.0, 0.0]]], np.float32)
    eye = np.eye(2, dtype=np.float32)[None]
    h = np.array([[0.0, 0.0], [5.0, 0.0], [-1.0, -1.0], [1e-30, 0.0]], np.float32)
    codes, _, _, best, second = o.projected_encode(h, eye, None, books, eye, None, normalize=True)
    # frame 2: u = -(1,1)/sqrt2, so |u|^2 = 1 and |u - v_0|^2 = |u - v_1|^2 = 2 + sqrt2;
    # frame 3: |e| = 1e-30 is floored to 1e-12, so u = (1e-18, 0) and the zero codeword is at 1e-36
    np.testing.assert_array_equal(codes[:, 0], [2, 0, 2, 2])
    np.testing.assert_allclose(best[:, 0], [0.0, 0.0, 1.0, 1e-36], rtol=1e-7, atol=0)
    np.testing.assert_allclose(second[:, 0], [1.0, 1.0, 2.0 + np.sqrt(2.0), 1.0], rtol=1e-15, atol=0)


ALL_PINS = [
    pin_handworked,
    pin_decode_order,
    pin_single_stage_cdist,
    pin_every_stage_cdist,
    pin_constructed_recovery,
    pin_best_is_residual_norm,
    pin_integer_exact,
    pin_prefix_and_permutation,
    pin_decode_gather,
    pin_linear,
    pin_projected_handworked,
    pin_projected_identity_is_plain_rvq,
    pin_projected_integer_exact,
    pin_projected_follows_given_encodings,
    pin_projected_prefix_and_decode,
    pin_cosine_handworked,
    pin_cosine_against_cdist,
    pin_cosine_norm_floor,
]
