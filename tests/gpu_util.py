"""Shared helpers for the GPU parity tests (HIP path vs CPU oracle)."""

import os

import numpy as np
import pytest
import torch

import oracle
import stage_dump

HAS_GPU = torch.cuda.is_available()
needs_gpu = pytest.mark.skipif(not HAS_GPU, reason="no GPU visible")
DEV = torch.device("cuda:0") if HAS_GPU else None


def rvq():
    """The HIP binding; raises (fails the test) if librvq.so is missing where a GPU is present."""
    import residual_vector_quantization_amd as m
    m.load()
    return m


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return None if t is None else t.cpu().numpy()


def announce(what, **shape):
    """Prints (and flushes) what the next GPU step runs, so a hang names its case."""
    print(f"[gpu case] {what} " + " ".join(f"{k}={v}" for k, v in shape.items()), flush=True)


SCORINGS = ["default", "fp32", "prepared"]

# Batches of up to 16384 frames (8192 with prepared codebooks) take a
# split-codebook encode (one 32-frame tile per workgroup, the codebook split
# over its wavefronts); larger ones a wide kernel. widen() embeds a small
# case into a batch that takes the wide kernel on every path.
SPLIT_MAX_FRAMES = 16384
PREPARED_SPLIT_MAX_FRAMES = 8192
WIDE_FRAMES = SPLIT_MAX_FRAMES + 300


def widen(x, seed=0):
    """(x_wide, idx): x followed by N(0,1) filler frames up to WIDE_FRAMES; idx selects x's frames
    and the batch's last 32 frames (its ragged tail) for the oracle comparison."""
    n = x.shape[0]
    fill = np.random.default_rng(seed + 7777).standard_normal((WIDE_FRAMES - n, x.shape[1])).astype(np.float32)
    xw = np.concatenate([x, fill], axis=0)
    idx = np.unique(np.concatenate([np.arange(n), np.arange(WIDE_FRAMES - 32, WIDE_FRAMES)]))
    return xw, idx


def check_encode(x, books, n_stages=None, idx=None, roundtrip=True, scoring="default"):
    """Runs the HIP encode (and roundtrip) and compares with the oracle.

    ``scoring`` "default" goes through rvq_encode / rvq_roundtrip, any other
    value through rvq_encode_scored. ``idx``: compare only those frames (the
    oracle runs on x[idx]); the GPU still encodes every frame. Codes must be
    identical; residual and recon bit-identical (they are deterministic
    float32 functions of the codes). Returns a small report dict.
    """
    m = rvq()
    q = books.shape[0] if n_stages is None else n_stages
    announce("encode", n=x.shape[0], q=q, k=books.shape[1], scoring=scoring)
    xg, bg = to_dev(x), to_dev(books)
    prep = m.rvq_prepare_codebooks(bg) if scoring == "prepared" else None
    if scoring == "default":
        codes, res = m.rvq_encode(xg, bg, n_stages=q)
    elif scoring == "prepared":
        codes, _, res = m.rvq_encode_prepared(xg, bg, prep, n_stages=q)
    else:
        codes, _, res = m.rvq_encode_scored(xg, bg, scoring, n_stages=q, recon=False)
    if roundtrip:
        if scoring == "default":
            codes2, recon, res2 = m.rvq_roundtrip(xg, bg, n_stages=q)
        elif scoring == "prepared":
            codes2, recon, res2 = m.rvq_encode_prepared(xg, bg, prep, n_stages=q, recon=True)
        else:
            codes2, recon, res2 = m.rvq_encode_scored(xg, bg, scoring, n_stages=q)
        out = m.rvq_decode(codes2, bg)
    torch.cuda.synchronize()
    codes, res = host(codes), host(res)
    sel = np.arange(x.shape[0]) if idx is None else idx
    oc, ores, best, second = oracle.get().encode(x[sel], books, n_stages=q)
    gc = codes[sel]
    mism = (gc != oc).any(axis=1)
    ties = oracle.near_tie(best, second)
    if os.environ.get("RVQ_DUMP"):   # per-stage dump before any assertion
        test = os.environ.get("PYTEST_CURRENT_TEST", "encode").split(" ")[0]
        stage_dump.write(os.environ["RVQ_DUMP"], f"{test}_{scoring}", sel, gc, oc, best, second, ties)
    report = {"frames": int(sel.size), "mismatch_frames": int(mism.sum()),
              "near_tie_frames": int(ties.any(axis=1).sum())}
    if mism.any():
        bad = np.nonzero(mism)[0]
        first = np.argmax(gc[bad] != oc[bad], axis=1)
        exempt = ties[bad, first]
        report["mismatch_exempt"] = int(exempt.sum())
        report["first_bad"] = [(int(sel[b]), int(s), int(gc[b, s]), int(oc[b, s]),
                                float(best[b, s]), float(second[b, s])) for b, s in zip(bad[:5], first[:5])]
    assert not mism.any(), f"codes differ from the oracle: {report}"
    assert gc.min() >= 0 and gc.max() < books.shape[1]
    np.testing.assert_array_equal(res[sel], ores)
    if roundtrip:
        codes2, recon, res2, out = host(codes2), host(recon), host(res2), host(out)
        np.testing.assert_array_equal(codes2, codes)
        np.testing.assert_array_equal(res2, res)
        np.testing.assert_array_equal(recon, out)
        orec = oracle.get().decode(oc, books[:q])
        np.testing.assert_array_equal(recon[sel], orec)
    return report
