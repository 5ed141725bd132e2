"""GPU parity of rvq_project_roundtrip (fc -> encode -> decode -> fc2), stage by stage.

(i) the GPU's latent against the oracle's float64 linear layer, within 1e-5
of each frame's norm; (ii) the GPU's codes and latent_recon against the
oracle run on the GPU's own latent, bit for bit (fp32 GEMM rounding can move
a frame across a near-tie, so the quantizer is judged on the input it was
given); (iii) the GPU's h_recon against the oracle's linear layer applied to
the GPU's latent_recon, within 1e-5 of each frame's norm.
"""

import numpy as np
import pytest

import oracle
import rvq_workloads as W
from gpu_util import needs_gpu, rvq, to_dev, host, announce

pytestmark = [pytest.mark.gpu, needs_gpu]

REL = 1e-5


def _rel_rows(a, b):
    num = np.linalg.norm(a.astype(np.float64) - b.astype(np.float64), axis=1)
    den = np.linalg.norm(b.astype(np.float64), axis=1)
    return num / np.maximum(den, 1e-30)


def check_project(h, w_in, b_in, books, w_out, b_out, idx=None, prepared=False):
    """``prepared``: pass rvq_prepare_codebooks' output (the encode then reads the prepared layout)."""
    m = rvq()
    announce("project_roundtrip", n=h.shape[0], hidden=h.shape[1], q=books.shape[0], prepared=prepared)
    dev = lambda a: None if a is None else to_dev(a)
    bg = to_dev(books)
    prep = m.rvq_prepare_codebooks(bg) if prepared else None
    codes, lat, lat_rec, h_rec = (host(t) for t in m.rvq_project_roundtrip(
        to_dev(h), to_dev(w_in), dev(b_in), bg, to_dev(w_out), dev(b_out), prepared=prep))
    sel = np.arange(h.shape[0]) if idx is None else idx
    o = oracle.get()
    y = o.linear(h[sel], w_in, b_in)
    r1 = _rel_rows(lat[sel], y)
    assert r1.max() <= REL, f"fc: max relative error {r1.max():.3g}"
    oc, _, _, _ = o.encode(lat[sel], books)
    np.testing.assert_array_equal(codes[sel], oc)
    np.testing.assert_array_equal(lat_rec[sel], o.decode(oc, books))
    hr = o.linear(lat_rec[sel], w_out, b_out)
    r3 = _rel_rows(h_rec[sel], hr)
    assert r3.max() <= REL, f"fc2: max relative error {r3.max():.3g}"
    return float(r1.max()), float(r3.max())


@pytest.mark.parametrize("prepared", [False, True])
@pytest.mark.parametrize("n,hidden,bias", [(677, 1024, True), (300, 1024, False), (129, 192, True),
                                           (1, 64, True), (16500, 128, True), (5, 1024, True), (40, 512, False),
                                           (100, 2048, True), (9000, 512, True)])
def test_project_small(n, hidden, bias, prepared):
    rng = np.random.default_rng(n + hidden)
    h = rng.standard_normal((n, hidden)).astype(np.float32)
    w_in = (rng.standard_normal((64, hidden)) / np.sqrt(hidden)).astype(np.float32)
    w_out = (rng.standard_normal((hidden, 64)) / 8.0).astype(np.float32)
    b_in = rng.standard_normal(64).astype(np.float32) if bias else None
    b_out = rng.standard_normal(hidden).astype(np.float32) if bias else None
    books = (rng.standard_normal((8, 1024, 64)) * 0.5 ** np.arange(8)[:, None, None]).astype(np.float32)
    e1, e3 = check_project(h, w_in, b_in, books, w_out, b_out, prepared=prepared)
    announce("project errors", fc=e1, fc2=e3)


@pytest.mark.parametrize("prepared", [False, True])
def test_project_full_size_sampled(prepared):
    w = W.WORKLOADS["projected"]
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    w_in, b_in, w_out, b_out = W.projection_weights(w)
    h = W.hidden_states(w)
    idx = W.sample_frames(w.n_frames, 2048, seed=4)
    e1, e3 = check_project(h, w_in, b_in, books, w_out, b_out, idx=idx, prepared=prepared)
    announce("project full-size errors", fc=e1, fc2=e3)


def test_project_unsupported_hidden():
    import torch
    m = rvq()
    d = "cuda:0"
    with pytest.raises(m.RVQError) as e:
        m.rvq_project_roundtrip(torch.zeros((4, 100), device=d), torch.zeros((64, 100), device=d), None,
                                torch.zeros((2, 64, 64), device=d), torch.zeros((100, 64), device=d), None)
    assert e.value.status == m.RVQ_ERR_UNSUPPORTED


# fc2 scales each frame's 64 values and each 32-row weight tile by a power of
# two before its fp16 split, and undoes both in the bias step (one fused
# multiply-add while the combined factor is a float, two steps otherwise).
# Codebooks and fc2 weights far from 1 move the frame and tile exponents over
# their range; the first case takes the two-step path (a combined factor
# below 2^-149), the others the fused one at large exponents of either sign.
@pytest.mark.parametrize("book_scale,w_scale,bias", [(2.0 ** -60, 2.0 ** -64, False), (1.0, 2.0 ** -100, False),
                                                     (2.0 ** 40, 2.0 ** -40, True), (2.0 ** 50, 2.0 ** 50, False),
                                                     (2.0 ** -60, 2.0 ** -64, True)])
def test_project_fc2_scales(book_scale, w_scale, bias):
    rng = np.random.default_rng(17)
    n, hidden = 300, 1024
    h = rng.standard_normal((n, hidden)).astype(np.float32)
    w_in = (rng.standard_normal((64, hidden)) / np.sqrt(hidden)).astype(np.float32)
    books = (rng.standard_normal((4, 256, 64)) * 0.5 ** np.arange(4)[:, None, None] * book_scale).astype(np.float32)
    w_in = (w_in * np.float32(book_scale)).astype(np.float32)   # latents on the codebooks' scale
    w_out = (rng.standard_normal((hidden, 64)) / 8.0 * w_scale).astype(np.float32)
    b_out = (rng.standard_normal(hidden) * book_scale * w_scale).astype(np.float32) if bias else None
    e1, e3 = check_project(h, w_in, None, books, w_out, b_out)
    announce("project fc2-scale errors", fc=e1, fc2=e3)


def test_project_fc2_chunks():
    """More frames than one fc2 chunk (2^20 frames: read-ahead of the inputs, then the products), so the
    second chunk's offsets are exercised; sampled frames on both sides of the boundary and at the end."""
    rng = np.random.default_rng(23)
    n, hidden = (1 << 20) + 37, 512
    h = rng.standard_normal((n, hidden), dtype=np.float32)
    w_in = (rng.standard_normal((64, hidden)) / np.sqrt(hidden)).astype(np.float32)
    w_out = (rng.standard_normal((hidden, 64)) / 8.0).astype(np.float32)
    b_out = rng.standard_normal(hidden).astype(np.float32)
    books = (rng.standard_normal((4, 256, 64)) * 0.5 ** np.arange(4)[:, None, None]).astype(np.float32)
    edge = np.arange((1 << 20) - 40, n)
    idx = np.unique(np.concatenate([W.sample_frames(n, 512, seed=7), edge, [0, 1, 31, 32]]))
    e1, e3 = check_project(h, w_in, None, books, w_out, b_out, idx=idx, prepared=True)
    announce("project fc2-chunk errors", fc=e1, fc2=e3)
