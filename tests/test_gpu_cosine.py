"""GPU parity of the normalized (cosine) per-stage projected RVQ.

rvq_cosine_prepare / rvq_cosine_encode (with rvq_projected_prepare's 8-dim
table and rvq_projected_decode) against the oracle's normalized projected
encode, stage by stage:

(i)   unit codewords equal the float64 definition c / max(|c|, 1e-12)
      (squares summed in order) bit for bit; the table equals the oracle's
      float64 linear layer on every codeword bit for bit;
(ii)  the oracle, taking each stage's argmin on the GPU's own projection,
      returns the GPU's codes and final residual bit for bit;
(iii) every stage's projection is within 1e-5 of the norm of the oracle's
      float64 projection of the same residual;
(iv)  the decode equals the oracle's projected decode bit for bit;
(v)   end to end, disagreements with the oracle's own projections start only
      at near-ties.
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


def _units_f64(books):
    c = books.astype(np.float64)
    ss = c[..., 0] * c[..., 0]
    for j in range(1, c.shape[-1]):
        ss = ss + c[..., j] * c[..., j]
    return c / np.maximum(np.sqrt(ss), 1e-12)[..., None]


def _weights(rng, q, k, hidden, bias, decay=0.85):
    books = (rng.standard_normal((q, k, 8)) * decay ** np.arange(q)[:, None, None]).astype(np.float32)
    w_in = (rng.standard_normal((q, 8, hidden)) / np.sqrt(hidden)).astype(np.float32)
    w_out = (rng.standard_normal((q, hidden, 8)) / np.sqrt(8.0)).astype(np.float32)
    b_in = (0.05 * rng.standard_normal((q, 8))).astype(np.float32) if bias else None
    b_out = (0.05 * rng.standard_normal((q, hidden))).astype(np.float32) if bias else None
    return books, w_in, b_in, w_out, b_out


def check_cosine(h, books, w_in, b_in, w_out, b_out, idx=None, n_stages=None, codes_ld=None):
    m = rvq()
    q = books.shape[0] if n_stages is None else n_stages
    n, hidden = h.shape
    announce("cosine", n=n, hidden=hidden, q=q, k=books.shape[1])
    dev = lambda a: None if a is None else to_dev(a)
    bg = to_dev(books)
    units = m.rvq_cosine_prepare(bg)
    table = m.rvq_projected_prepare(bg, to_dev(w_out), dev(b_out))
    hg = to_dev(h)
    ld = q if codes_ld is None else codes_ld
    codes_buf = torch.full((n, ld), -7, dtype=torch.int32, device=hg.device)
    latent = torch.empty((q, n, 8), dtype=torch.float32, device=hg.device)
    residual = torch.empty_like(hg)
    m.rvq_cosine_encode(hg, to_dev(w_in), dev(b_in), units, table, n_stages=q, out=(codes_buf, latent, residual))
    recon = m.rvq_projected_decode(codes_buf, table, n_stages=q)
    torch.cuda.synchronize()
    codes_all, lat, res, rec = host(codes_buf), host(latent), host(residual), host(recon)
    if ld > q:
        assert (codes_all[:, q:] == -7).all(), "columns past n_stages were written"
    codes = codes_all[:, :q]
    o = oracle.get()
    np.testing.assert_array_equal(host(units), _units_f64(books))
    tab = host(table)
    for s in range(books.shape[0]):
        np.testing.assert_array_equal(tab[s], o.linear(books[s], w_out[s], None if b_out is None else b_out[s]))
    sel = np.arange(n) if idx is None else idx
    hs = h[sel]
    oc, oe, ores, _, _ = o.projected_encode(hs, w_in, b_in, books, w_out, b_out, n_stages=q,
                                            e_given=np.ascontiguousarray(lat[:, sel]), normalize=True)
    np.testing.assert_array_equal(codes[sel], oc)
    np.testing.assert_array_equal(res[sel], ores)
    rel = _rel_rows(lat[:, sel], oe)
    assert rel.max() <= REL, f"latent: max relative error {rel.max():.3g}"
    np.testing.assert_array_equal(rec[sel], o.projected_decode(codes[sel], books[:q], w_out, b_out))
    c_own, _, _, best, second = o.projected_encode(hs, w_in, b_in, books, w_out, b_out, n_stages=q, normalize=True)
    mism = (c_own != codes[sel]).any(axis=1)
    if mism.any():
        bad = np.nonzero(mism)[0]
        first = np.argmax(c_own[bad] != codes[sel][bad], axis=1)
        ties = oracle.near_tie(best, second)[bad, first]
        assert ties.all(), f"{int((~ties).sum())} frames differ first at a stage that is not a near-tie"
    return {"frames": int(sel.size), "latent_max_rel": float(rel.max()), "mismatch_frames": int(mism.sum())}


# codebooks of at most 1024 entries run all stages in one kernel; larger ones
# (1500, 2048 here) take one projection and one argmin launch per stage
@pytest.mark.parametrize("n,hidden,q,k,bias", [(1, 64, 1, 16, True), (63, 320, 4, 1000, True),
                                               (300, 1024, 32, 1024, True), (2000, 1024, 3, 1024, False),
                                               (129, 512, 8, 200, True), (700, 768, 5, 1024, True),
                                               (33, 256, 6, 1500, True), (500, 1024, 3, 2048, False)])
def test_cosine_small(n, hidden, q, k, bias):
    rng = np.random.default_rng(n * 5 + hidden + q + k)
    h = rng.standard_normal((n, hidden)).astype(np.float32)
    books, w_in, b_in, w_out, b_out = _weights(rng, q, k, hidden, bias)
    rep = check_cosine(h, books, w_in, b_in, w_out, b_out)
    announce("cosine report", **rep)


def test_cosine_ties_zeros_partial_depth():
    """Same-direction and duplicated codewords (exact ties), a zero codeword, zero projections."""
    rng = np.random.default_rng(51)
    q, k, hidden, n = 4, 256, 128, 400
    books, w_in, _, w_out, b_out = _weights(rng, q, k, hidden, False)
    books[:, 100:110] = books[:, 10:20] * 2.0     # same direction as a lower row: equal unit codewords
    books[:, 120:125] = books[:, 30:35]           # exact duplicates
    books[:, 5] = 0.0                              # zero codeword: unit vector 0
    h = rng.standard_normal((n, hidden)).astype(np.float32)
    h[:20] = 0.0                                   # zero projections at stage 0 (no bias)
    check_cosine(h, books, w_in, None, w_out, b_out, n_stages=3, codes_ld=6)
    m = rvq()
    bg = to_dev(books)
    codes, _, _ = m.rvq_cosine_encode(to_dev(h), to_dev(w_in), None, m.rvq_cosine_prepare(bg),
                                      m.rvq_projected_prepare(bg, to_dev(w_out), None))
    c = host(codes)
    assert not ((c >= 100) & (c < 110)).any() and not ((c >= 120) & (c < 125)).any()


def test_cosine_argument_errors():
    m = rvq()
    rng = np.random.default_rng(52)
    books, w_in, b_in, w_out, b_out = _weights(rng, 2, 64, 2048, True)
    bg = to_dev(books)
    units = m.rvq_cosine_prepare(bg)
    table = torch.zeros((2, 64, 2048), device=bg.device)
    with pytest.raises(m.RVQError) as e:
        m.rvq_cosine_encode(to_dev(np.zeros((4, 2048), np.float32)), to_dev(w_in), to_dev(b_in), units, table)
    assert e.value.status == m.RVQ_ERR_UNSUPPORTED


def test_cosine_full_size_sampled():
    """The benchmark's workload and launch configuration; oracle on a seeded frame sample."""
    w = W.WORKLOADS["cosine"]
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    w_in, b_in, w_out, b_out = W.stage_projection_weights(w)
    h = W.hidden_states(w)
    idx = W.sample_frames(w.n_frames, 1024, seed=9)
    rep = check_cosine(h, books, w_in, b_in, w_out, b_out, idx=idx)
    announce("cosine full-size report", **rep)
