"""Seeded synthetic inputs for residual vector quantization (RVQ).

This module only draws random numbers. It holds no step of the method:
no distance, no argmin, no residual update, no gather-sum. Both the CPU
oracle (under ``oracle/``) and the HIP path read their inputs from here,
so neither has to import the other.

Shapes follow the codec pages:

* "Architecture" (omnivoice.cpp), section "RVQ codec": 8 codebooks, each
  1024 entries of dimension 64, at 25 frames per second.
* "Maintainer's guide -- moss-tts.cpp", section "What this project is":
  32 RVQ code streams at 12.5 Hz.

No trained codec weights exist here, so every codebook, latent and
projection matrix is drawn from a seeded PCG64 generator. Each kind of
draw has its own stream, so changing one size never shifts another draw:

    codebook = 1, latents = 2, code indices = 3, noise = 4,
    fc (1024 -> 64) weights = 5, fc2 (64 -> 1024) weights = 6,
    per-stage project_in weights = 7, project_out weights = 8,
    project_in biases = 9, project_out biases = 10.

Readings of the recipe that the pages leave open:

* ``N(0, s)`` for additive noise names a standard deviation (sigma = 1e-3
  for the tiny round trip, 1e-2 for the batched set). Under a variance
  reading the tiny set's late stages would not be recoverable, which
  contradicts "well separated".
* ``N(0, 1/fan_in)`` for linear weights names a variance (std 1/32 for
  fc, 1/8 for fc2), the usual 1/fan_in scaling that keeps outputs near
  unit scale.
* Per-stage projections ("RVQ codec" section: project_in / project_out of
  every codebook, both with bias) use the same 1/fan_in variances; the
  pages give no values for their biases, so they are drawn small,
  N(0, 0.05^2), to exercise the bias path.
* The normalized quantizer ("Maintainer's guide -- moss-tts.cpp": 32
  codebooks at 12.5 Hz, 1024 entries each behind 1025-wide heads, 8-dim
  codebook space) takes a 1024-wide input here; the page does not state it.
* Frames built as "sums of random codewords plus noise" are summed in
  float64 and rounded once to float32. That is input synthesis, done at a
  higher precision than the method's own float32 arithmetic.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

STREAM_CODEBOOK = 1
STREAM_LATENTS = 2
STREAM_CODES = 3
STREAM_NOISE = 4
STREAM_FC_IN = 5
STREAM_FC_OUT = 6
STREAM_STAGE_IN = 7
STREAM_STAGE_OUT = 8
STREAM_STAGE_IN_BIAS = 9
STREAM_STAGE_OUT_BIAS = 10


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes plus the recipe of its inputs."""

    name: str
    n_frames: int
    n_stages: int          # Q
    n_codes: int           # K
    dim: int               # D
    decay: float           # codebook q is N(0,1) * decay**q
    constructed_from: int  # frames [constructed_from, N) are sums of codewords + noise
    noise_sigma: float     # std of the additive noise on constructed frames
    frame_rate_hz: float   # for seconds-of-audio figures
    hidden: int = 0        # >0: projected workload with fc hidden->dim and fc2 dim->hidden
    per_stage: bool = False  # projections per codebook (project_in / project_out) instead of fc / fc2
    normalized: bool = False  # argmin between unit-norm projection and unit-norm codewords
    seed: int = 0
    description: str = ""

    @property
    def projected(self) -> bool:
        return self.hidden > 0 and not self.per_stage


# The eight workloads. Sizes and recipes as the codec shapes dictate; the
# description strings state them for result lines.
WORKLOADS = {
    "tiny": Workload(
        "tiny", 25, 8, 1024, 64, 0.5, 0, 1e-3, 25.0,
        description="25 frames (1 s at 25 Hz); x = sum_q C[q,t_q] + N(0, sigma=1e-3); "
                    "C[q] ~ N(0,1)*0.5^q, Q=8, K=1024, D=64; seed 0"),
    "clip": Workload(
        "clip", 1500, 8, 1024, 64, 0.5, 1500, 0.0, 25.0,
        description="1500 frames (60 s at 25 Hz) x ~ N(0,1); C[q] ~ N(0,1)*0.5^q, "
                    "Q=8, K=1024, D=64; seed 0"),
    "batched": Workload(
        "batched", 192_000, 8, 1024, 64, 0.5, 96_000, 1e-2, 25.0,
        description="256 clips x 750 frames = 192000 frames; frames 0..95999 ~ N(0,1), "
                    "frames 96000..191999 = sum_q C[q,t_q] + N(0, sigma=1e-2); "
                    "C[q] ~ N(0,1)*0.5^q, Q=8, K=1024, D=64; seed 0"),
    "deep": Workload(
        "deep", 720_000, 32, 1024, 64, 0.85, 720_000, 0.0, 12.5,
        description="16 clips x 45000 frames (1 h at 12.5 Hz) = 720000 frames ~ N(0,1); "
                    "C[q] ~ N(0,1)*0.85^q, Q=32, K=1024, D=64; seed 0"),
    "large": Workload(
        "large", 192_000, 10, 4096, 64, 0.5, 192_000, 0.0, 44100.0 / 2048.0,
        description="96 clips x 2000 frames = 192000 frames (44.1 kHz, 2048 samples per frame) "
                    "~ N(0,1); C[q] ~ N(0,1)*0.5^q, Q=10, K=4096, D=64 (codebook dim assumed); "
                    "seed 0"),
    "projected": Workload(
        "projected", 1_000_000, 8, 1024, 64, 0.5, 1_000_000, 0.0, 25.0, hidden=1024,
        description="1e6 hidden vectors [1e6,1024] ~ N(0,1); fc 1024->64 W ~ N(0, var 1/1024), "
                    "b = 0; RVQ Q=8, K=1024, D=64, C[q] ~ N(0,1)*0.5^q; fc2 64->1024 "
                    "W ~ N(0, var 1/64), b = 0; seed 0"),
    "stage_projected": Workload(
        "stage_projected", 192_000, 8, 1024, 64, 0.5, 192_000, 0.0, 25.0, hidden=1024, per_stage=True,
        description="256 clips x 750 frames = 192000 hidden vectors [N,1024] ~ N(0,1); per stage q < 8: "
                    "project_in W_in[q] [64,1024] ~ N(0, var 1/1024), b_in[q] ~ N(0, 0.05^2); "
                    "C[q] [1024,64] ~ N(0,1)*0.5^q; project_out W_out[q] [1024,64] ~ N(0, var 1/64), "
                    "b_out[q] ~ N(0, 0.05^2); seed 0"),
    "cosine": Workload(
        "cosine", 180_000, 32, 1024, 8, 0.85, 180_000, 0.0, 12.5, hidden=1024, per_stage=True, normalized=True,
        description="16 clips x 11250 frames (4 h at 12.5 Hz) = 180000 hidden vectors [N,1024] ~ N(0,1) "
                    "(input width assumed); per stage q < 32: project_in W_in[q] [8,1024] ~ N(0, var 1/1024), "
                    "b_in[q] ~ N(0, 0.05^2); C[q] [1024,8] ~ N(0,1)*0.85^q; project_out W_out[q] [1024,8] "
                    "~ N(0, var 1/8), b_out[q] ~ N(0, 0.05^2); argmin on unit-norm projection and codewords; "
                    "seed 0"),
}


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def codebooks(n_stages: int, n_codes: int, dim: int, decay: float, seed: int = 0) -> np.ndarray:
    """[Q, K, D] float32 codebooks; stage q is N(0,1) * decay**q, drawn in float64."""
    g = _rng(seed, STREAM_CODEBOOK)
    c = g.standard_normal((n_stages, n_codes, dim))
    c *= (decay ** np.arange(n_stages, dtype=np.float64))[:, None, None]
    return c.astype(np.float32)


def _normal_f32(g: np.random.Generator, rows: int, cols: int, chunk_rows: int = 1 << 18) -> np.ndarray:
    """N(0,1) float32 [rows, cols], drawn in row chunks to bound host memory."""
    out = np.empty((rows, cols), dtype=np.float32)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        g.standard_normal((r1 - r0, cols), dtype=np.float32, out=out[r0:r1])
    return out


def latents(w: Workload, cb: Optional[np.ndarray] = None):
    """Latents x [N, D] float32 for workload ``w`` (non-projected workloads).

    Returns ``(x, t)``: ``t`` [N, Q] int32 holds the codeword indices used to
    build frames ``[w.constructed_from, N)`` and -1 elsewhere.
    """
    if cb is None:
        cb = codebooks(w.n_stages, w.n_codes, w.dim, w.decay, w.seed)
    n, nb = w.n_frames, w.constructed_from
    x = np.empty((n, w.dim), dtype=np.float32)
    if nb > 0:
        x[:nb] = _normal_f32(_rng(w.seed, STREAM_LATENTS), nb, w.dim)
    t = np.full((n, w.n_stages), -1, dtype=np.int32)
    m = n - nb
    if m > 0:
        tc = _rng(w.seed, STREAM_CODES).integers(0, w.n_codes, size=(m, w.n_stages), dtype=np.int64)
        acc = np.zeros((m, w.dim), dtype=np.float64)
        for q in range(w.n_stages):
            acc += cb[q][tc[:, q]].astype(np.float64)
        acc += w.noise_sigma * _rng(w.seed, STREAM_NOISE).standard_normal((m, w.dim))
        x[nb:] = acc.astype(np.float32)
        t[nb:] = tc.astype(np.int32)
    return x, t


def projection_weights(w: Workload):
    """fc weight [D, H] (var 1/H) and fc2 weight [H, D] (var 1/D), PyTorch (out, in) order.

    Both biases are zero; they are returned as explicit zero vectors.
    """
    h, d = w.hidden, w.dim
    w_in = (_rng(w.seed, STREAM_FC_IN).standard_normal((d, h)) * (1.0 / np.sqrt(h))).astype(np.float32)
    w_out = (_rng(w.seed, STREAM_FC_OUT).standard_normal((h, d)) * (1.0 / np.sqrt(d))).astype(np.float32)
    return w_in, np.zeros(d, np.float32), w_out, np.zeros(h, np.float32)


def stage_projection_weights(w: Workload):
    """Per-stage projections, PyTorch (out, in) order, stacked over the Q stages:
    ``w_in`` [Q, D, H] (var 1/H), ``b_in`` [Q, D], ``w_out`` [Q, H, D] (var 1/D),
    ``b_out`` [Q, H]; biases N(0, 0.05^2)."""
    q, h, d = w.n_stages, w.hidden, w.dim
    w_in = (_rng(w.seed, STREAM_STAGE_IN).standard_normal((q, d, h)) * (1.0 / np.sqrt(h))).astype(np.float32)
    w_out = (_rng(w.seed, STREAM_STAGE_OUT).standard_normal((q, h, d)) * (1.0 / np.sqrt(d))).astype(np.float32)
    b_in = (0.05 * _rng(w.seed, STREAM_STAGE_IN_BIAS).standard_normal((q, d))).astype(np.float32)
    b_out = (0.05 * _rng(w.seed, STREAM_STAGE_OUT_BIAS).standard_normal((q, h))).astype(np.float32)
    return w_in, b_in, w_out, b_out


def hidden_states(w: Workload, rows: Optional[int] = None) -> np.ndarray:
    """Projected workload input h [N, H] float32 ~ N(0,1) (first ``rows`` rows if given)."""
    n = w.n_frames if rows is None else rows
    return _normal_f32(_rng(w.seed, STREAM_LATENTS), n, w.hidden)


def random_codes(n_frames: int, n_stages: int, n_codes: int, seed: int = 0) -> np.ndarray:
    """Uniform valid codes [N, Q] int32 (for decode-only cases)."""
    return _rng(seed, STREAM_CODES).integers(0, n_codes, size=(n_frames, n_stages), dtype=np.int64).astype(np.int32)


def sample_frames(n_frames: int, count: int, seed: int = 0) -> np.ndarray:
    """Sorted, seeded frame indices for sampled parity at full size.

    Always holds the first and last 64 frames (first tile, ragged tail) plus a
    uniform sample of the rest.
    """
    if count >= n_frames:
        return np.arange(n_frames, dtype=np.int64)
    edge = min(64, n_frames // 2)
    fixed = np.concatenate([np.arange(edge), np.arange(n_frames - edge, n_frames)])
    rest = _rng(seed, 99).choice(n_frames, size=max(0, count - fixed.size), replace=False)
    return np.unique(np.concatenate([fixed, rest])).astype(np.int64)
