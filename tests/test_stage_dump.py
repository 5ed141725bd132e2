"""The per-stage dump of the parity harness (RVQ_DUMP): what it records about a divergence."""

import numpy as np

import oracle
import rvq_workloads as W
import stage_dump


def test_dump_locates_first_divergent_stage(tmp_path):
    w = W.WORKLOADS["tiny"]
    books = W.codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    x, _ = W.latents(w, books)
    oc, _, best, second = oracle.get().encode(x, books)
    ties = oracle.near_tie(best, second)
    gc = oc.copy()
    gc[3, 2] = (gc[3, 2] + 1) % w.n_codes      # frame 3 first differs at stage 2
    gc[3, 5] = (gc[3, 5] + 7) % w.n_codes      # later stages may differ too
    gc[10, 0] = (gc[10, 0] + 1) % w.n_codes    # frame 10 at stage 0
    frames = np.arange(x.shape[0])
    path = stage_dump.write(str(tmp_path), "tests/x.py::case[a b]", frames, gc, oc, best, second, ties)
    assert path.endswith(".npz")
    # a second dump of the same name does not overwrite the first
    path2 = stage_dump.write(str(tmp_path), "tests/x.py::case[a b]", frames, oc, oc, best, second, ties)
    assert path2 != path
    with np.load(path) as z:
        fd = z["first_diff"]
        assert fd[3] == 2 and fd[10] == 0
        assert (np.delete(fd, [3, 10]) == -1).all()
        np.testing.assert_array_equal(z["oracle_codes"], oc)
        np.testing.assert_array_equal(z["gpu_codes"], gc)
        np.testing.assert_array_equal(z["best"], best)
        np.testing.assert_array_equal(z["near_tie"], ties)
    rep = stage_dump.summarize(path)
    assert rep["frames"] == x.shape[0] and rep["differing_frames"] == 2
    assert rep["differing_at_near_tie"] == int(ties[3, 2]) + int(ties[10, 0])
    assert stage_dump.summarize(path2)["differing_frames"] == 0
