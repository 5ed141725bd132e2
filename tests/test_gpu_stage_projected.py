"""GPU parity of the per-stage projected RVQ (rvq_projected_prepare / _encode / _decode).

Checked stage by stage against the oracle:

(i)   the table of projected codewords equals the oracle's float64 linear
      layer applied to every codeword, bit for bit;
(ii)  the oracle, taking each stage's argmin on the GPU's own latent
      (fp32 matrix-core GEMM rounding can move a frame across a near-tie),
      returns the GPU's codes and the GPU's final residual bit for bit;
(iii) the GPU's latent of every stage is within 1e-5 of the norm of the
      oracle's float64 projection of the same residual;
(iv)  the decode equals the oracle's projected decode of the GPU codes bit
      for bit;
(v)   end to end, the oracle on its own projections disagrees with the GPU
      codes only where the first differing stage is a near-tie.
"""

import numpy as np
import pytest
import torch

import oracle
import rvq_workloads as W
from gpu_util import needs_gpu, rvq, to_dev, host, announce

pytestmark = [pytest.mark.gpu, needs_gpu]

REL = 1e-5


def _rel_rows(a, b):
    num = np.linalg.norm(a.astype(np.float64) - b.astype(np.float64), axis=-1)
    den = np.linalg.norm(b.astype(np.float64), axis=-1)
    return num / np.maximum(den, 1e-30)


def _weights(rng, q, k, hidden, bias, decay=0.5):
    books = (rng.standard_normal((q, k, 64)) * decay ** np.arange(q)[:, None, None]).astype(np.float32)
    w_in = (rng.standard_normal((q, 64, hidden)) / np.sqrt(hidden)).astype(np.float32)
    w_out = (rng.standard_normal((q, hidden, 64)) / 8.0).astype(np.float32)
    b_in = (0.05 * rng.standard_normal((q, 64))).astype(np.float32) if bias else None
    b_out = (0.05 * rng.standard_normal((q, hidden))).astype(np.float32) if bias else None
    return books, w_in, b_in, w_out, b_out


def check_stage_projected(h, books, w_in, b_in, w_out, b_out, idx=None, n_stages=None, codes_ld=None,
                          in_place=False, prepared=False):
    """``prepared``: pass rvq_prepare_codebooks' output, so that every stage's argmin reads its block."""
    m = rvq()
    q = books.shape[0] if n_stages is None else n_stages
    n, hidden = h.shape
    announce("stage_projected", n=n, hidden=hidden, q=q, k=books.shape[1], in_place=in_place, prepared=prepared)
    dev = lambda a: None if a is None else to_dev(a)
    bg, wo, bo = to_dev(books), to_dev(w_out), dev(b_out)
    table = m.rvq_projected_prepare(bg, wo, bo)
    hg = to_dev(h)
    ld = q if codes_ld is None else codes_ld
    codes_buf = torch.full((n, ld), -7, dtype=torch.int32, device=hg.device)
    latent = torch.empty((q, n, 64), dtype=torch.float32, device=hg.device)
    residual = hg if in_place else torch.empty_like(hg)
    prep = m.rvq_prepare_codebooks(bg) if prepared else None
    m.rvq_projected_encode(hg, to_dev(w_in), dev(b_in), bg, table, n_stages=q, out=(codes_buf, latent, residual),
                           prepared=prep)
    recon = m.rvq_projected_decode(codes_buf, table, n_stages=q)
    torch.cuda.synchronize()
    codes_all, lat, res, rec, tab = host(codes_buf), host(latent), host(residual), host(recon), host(table)
    if ld > q:
        assert (codes_all[:, q:] == -7).all(), "columns past n_stages were written"
    codes = codes_all[:, :q]
    o = oracle.get()
    # (i) table
    for s in range(books.shape[0]):
        np.testing.assert_array_equal(tab[s], o.linear(books[s], w_out[s], None if b_out is None else b_out[s]))
    sel = np.arange(n) if idx is None else idx
    hs = h[sel]
    # (ii), (iii): the oracle follows the GPU's latent
    oc, oe, ores, _, _ = o.projected_encode(hs, w_in, b_in, books, w_out, b_out, n_stages=q,
                                            e_given=np.ascontiguousarray(lat[:, sel]))
    np.testing.assert_array_equal(codes[sel], oc)
    np.testing.assert_array_equal(res[sel], ores)
    rel = _rel_rows(lat[:, sel], oe)
    assert rel.max() <= REL, f"latent: max relative error {rel.max():.3g}"
    # (iv) decode
    np.testing.assert_array_equal(rec[sel], o.projected_decode(codes[sel], books[:q], w_out, b_out))
    # (v) end to end on the oracle's own projections
    c_own, _, _, best, second = o.projected_encode(hs, w_in, b_in, books, w_out, b_out, n_stages=q)
    mism = (c_own != codes[sel]).any(axis=1)
    if mism.any():
        bad = np.nonzero(mism)[0]
        first = np.argmax(c_own[bad] != codes[sel][bad], axis=1)
        ties = oracle.near_tie(best, second)[bad, first]
        assert ties.all(), f"{int((~ties).sum())} frames differ first at a stage that is not a near-tie"
    return {"frames": int(sel.size), "latent_max_rel": float(rel.max()), "mismatch_frames": int(mism.sum())}


@pytest.mark.parametrize("prepared", [False, True])
@pytest.mark.parametrize("n,hidden,q,k,bias", [(1, 64, 1, 64, True), (31, 192, 3, 100, True),
                                               (129, 1024, 8, 1024, True), (677, 1024, 2, 1000, False),
                                               (1000, 320, 5, 257, True), (257, 64, 8, 1024, False)])
def test_stage_projected_small(n, hidden, q, k, bias, prepared):
    rng = np.random.default_rng(n * 3 + hidden + q + k)
    h = rng.standard_normal((n, hidden)).astype(np.float32)
    books, w_in, b_in, w_out, b_out = _weights(rng, q, k, hidden, bias)
    rep = check_stage_projected(h, books, w_in, b_in, w_out, b_out, prepared=prepared)
    announce("stage_projected report", **rep)


def test_stage_projected_partial_depth_ld_and_in_place():
    rng = np.random.default_rng(41)
    h = rng.standard_normal((300, 256)).astype(np.float32)
    books, w_in, b_in, w_out, b_out = _weights(rng, 6, 512, 256, True)
    check_stage_projected(h, books, w_in, b_in, w_out, b_out, n_stages=4, codes_ld=7)
    check_stage_projected(h, books, w_in, b_in, w_out, b_out, n_stages=4, codes_ld=7, prepared=True)
    check_stage_projected(h, books, w_in, b_in, w_out, b_out, in_place=True)
    check_stage_projected(h, books, w_in, b_in, w_out, b_out, in_place=True, prepared=True)


def test_stage_projected_identity_is_plain_rvq():
    """hidden = 64 with identity projections and no biases gives the plain encode's codes and residual."""
    rng = np.random.default_rng(42)
    q, k, n = 4, 1024, 500
    books = (rng.standard_normal((q, k, 64)) * 0.5 ** np.arange(q)[:, None, None]).astype(np.float32)
    x = rng.standard_normal((n, 64)).astype(np.float32)
    eye = np.ascontiguousarray(np.broadcast_to(np.eye(64, dtype=np.float32), (q, 64, 64)))
    m = rvq()
    bg = to_dev(books)
    table = m.rvq_projected_prepare(bg, to_dev(eye))
    codes, lat, res = m.rvq_projected_encode(to_dev(x), to_dev(eye), None, bg, table)
    c0, r0 = m.rvq_encode(to_dev(x), bg)
    np.testing.assert_array_equal(host(codes), host(c0))
    np.testing.assert_array_equal(host(res), host(r0))
    np.testing.assert_array_equal(host(lat[0]), x)
    np.testing.assert_array_equal(host(m.rvq_projected_decode(codes, table)), host(m.rvq_decode(codes, bg)))


# tables of 4 MiB and more (with hidden <= 1024) take the stage-ordered decode
@pytest.mark.parametrize("n,hidden,q,k", [(40, 192, 3, 128), (41, 1024, 4, 1024), (203, 448, 9, 300),
                                          (37, 1280, 2, 1024)])
def test_stage_projected_decode_bad_codes(n, hidden, q, k):
    rng = np.random.default_rng(43 + n)
    books, _, _, w_out, b_out = _weights(rng, q, k, hidden, True)
    m = rvq()
    announce("projected decode", n=n, hidden=hidden, q=q, k=k)
    table = m.rvq_projected_prepare(to_dev(books), to_dev(w_out), to_dev(b_out))
    codes = W.random_codes(n, q, k, seed=5)
    codes[4, 1] = k
    codes[9, q - 1] = -1
    codes[n - 1, 0] = k + 7
    bad = [4, 9, n - 1]
    out = host(m.rvq_projected_decode(to_dev(codes), table))
    assert np.isnan(out[bad]).all()
    good = np.setdiff1d(np.arange(n), bad)
    np.testing.assert_array_equal(out[good], oracle.get().projected_decode(codes[good], books, w_out, b_out))


def test_stage_projected_empty_and_errors():
    m = rvq()
    rng = np.random.default_rng(44)
    books, w_in, b_in, w_out, b_out = _weights(rng, 2, 64, 128, True)
    bg = to_dev(books)
    table = m.rvq_projected_prepare(bg, to_dev(w_out), to_dev(b_out))
    codes, lat, res = m.rvq_projected_encode(to_dev(np.zeros((0, 128), np.float32)), to_dev(w_in), to_dev(b_in),
                                             bg, table)
    assert codes.shape == (0, 2) and res.shape == (0, 128)
    with pytest.raises(m.RVQError) as e:
        m.rvq_projected_prepare(bg, to_dev(np.zeros((2, 100, 64), np.float32)))
    assert e.value.status == m.RVQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("prepared", [False, True])
def test_stage_projected_full_size_sampled(prepared):
    """The benchmark's workload (which passes prepared codebooks); oracle on a seeded frame sample."""
    w = W.WORKLOADS["stage_projected"]
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    w_in, b_in, w_out, b_out = W.stage_projection_weights(w)
    h = W.hidden_states(w)
    idx = W.sample_frames(w.n_frames, 2048, seed=7)
    rep = check_stage_projected(h, books, w_in, b_in, w_out, b_out, idx=idx, prepared=prepared)
    announce("stage_projected full-size report", **rep)
