"""Per-stage dump of an encode parity comparison, for dump-and-diff debugging.

With ``RVQ_DUMP=<directory>`` in the environment, every encode comparison of
the GPU parity tests (``gpu_util.check_encode``) writes one ``.npz`` file
there before it asserts anything, so a failing comparison leaves its
evidence behind:

- ``frames``        [F]    batch indices of the compared frames
- ``gpu_codes``     [F, Q] codes from the HIP path
- ``oracle_codes``  [F, Q] codes from the float64 oracle
- ``best``, ``second`` [F, Q] the oracle's smallest and second-smallest
  distance per stage (float64)
- ``near_tie``      [F, Q] the oracle's near-tie flag per stage
- ``first_diff``    [F]    first stage where the two code rows differ, -1 if none

Later stages legitimately diverge once a stage differs (the residuals differ),
so ``first_diff`` is the stage to look at, and ``near_tie[f, first_diff[f]]``
says whether that difference is an allowed near-tie.
"""

import os
import re

import numpy as np


def first_divergence(gpu_codes, oracle_codes):
    """Index of the first stage where each frame's codes differ, -1 where they agree."""
    diff = np.asarray(gpu_codes) != np.asarray(oracle_codes)
    return np.where(diff.any(axis=1), np.argmax(diff, axis=1), -1)


def write(directory, name, frames, gpu_codes, oracle_codes, best, second, near_tie):
    """Writes one comparison to ``directory/<name>.npz`` (name made file-safe, numbered if taken)."""
    os.makedirs(directory, exist_ok=True)
    base = re.sub(r"[^A-Za-z0-9_.-]+", "_", name).strip("_") or "encode"
    path = os.path.join(directory, base + ".npz")
    n = 1
    while os.path.exists(path):
        path = os.path.join(directory, f"{base}_{n}.npz")
        n += 1
    np.savez(path, frames=np.asarray(frames), gpu_codes=np.asarray(gpu_codes),
             oracle_codes=np.asarray(oracle_codes), best=np.asarray(best), second=np.asarray(second),
             near_tie=np.asarray(near_tie), first_diff=first_divergence(gpu_codes, oracle_codes))
    return path


def summarize(path):
    """What a dump says: frames compared, frames that differ, and how many of those differ first at a
    near-tie stage."""
    with np.load(path) as z:
        fd = z["first_diff"]
        bad = np.nonzero(fd >= 0)[0]
        return {"frames": int(fd.size), "differing_frames": int(bad.size),
                "differing_at_near_tie": int(z["near_tie"][bad, fd[bad]].sum()) if bad.size else 0}
