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
* linear layer against numpy's float64 matmul.
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
]
