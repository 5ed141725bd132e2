"""CPU oracle for residual vector quantization -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product.

The arithmetic lives in ``rvq_oracle.c`` (plain C, float64 distances); this
module compiles it with gcc and marshals numpy arrays through ctypes.

Pinned by ``tests/test_oracle_pins.py`` against: a hand-worked example
(``tests/golden/``), scipy's ``cdist`` 1-nearest-neighbour for one stage,
exact recovery of codes from well-separated constructed inputs, exact
integer arithmetic with deliberate ties, the identity "best distance of the
last stage equals the squared norm of the final residual", and invariants
(prefix consistency, batch permutation, optimality of every stage's pick).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "rvq_oracle.c")
LIBRARY = os.path.join(_HERE, "_build", "librvq_oracle.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror", "-pthread"]


def build(source: str = SOURCE, out: str = LIBRARY, werror: bool = True) -> str:
    """Compiles the oracle with gcc (always; cheap) and returns the library path."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    flags = [f for f in CFLAGS if werror or f != "-Werror"]
    subprocess.run(["gcc", *flags, source, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_F32P = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_F64P = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_I32P = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")


class Oracle:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_encode.restype = ctypes.c_int
        lib.oracle_encode.argtypes = [
            _F32P, ctypes.c_int64, ctypes.c_int32, _F32P, ctypes.c_int32, ctypes.c_int32,
            _I32P, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [
            _I32P, ctypes.c_int32, ctypes.c_int64, _F32P, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, _F32P, ctypes.c_int]
        lib.oracle_linear.restype = ctypes.c_int
        lib.oracle_linear.argtypes = [
            _F32P, ctypes.c_int64, ctypes.c_int32, _F32P, ctypes.c_void_p, ctypes.c_int32,
            _F32P, ctypes.c_int]
        lib.oracle_projected_encode.restype = ctypes.c_int
        lib.oracle_projected_encode.argtypes = [
            _F32P, ctypes.c_int64, ctypes.c_int32, _F32P, ctypes.c_void_p, _F32P, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, _F32P, ctypes.c_void_p, ctypes.c_void_p, _I32P,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int]
        lib.oracle_projected_decode.restype = ctypes.c_int
        lib.oracle_projected_decode.argtypes = [
            _I32P, ctypes.c_int32, ctypes.c_int64, _F32P, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, _F32P, ctypes.c_void_p, ctypes.c_int32, _F32P, ctypes.c_int]
        self.lib = lib
        self.last_threads = 0

    @staticmethod
    def _ptr(a: Optional[np.ndarray]):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    def encode(self, x: np.ndarray, books: np.ndarray, n_stages: Optional[int] = None,
               threads: int = 0):
        """Greedy residual encode.

        ``x`` [N, D] float32, ``books`` [Q, K, D] float32. Uses the first
        ``n_stages`` stages (all by default). Returns ``(codes [N, Q] int32,
        residual [N, D] float32, best [N, Q] float64, second [N, Q] float64)``
        where ``best``/``second`` are each stage's smallest and second
        smallest squared distance.
        """
        x = np.ascontiguousarray(x, dtype=np.float32)
        books = np.ascontiguousarray(books, dtype=np.float32)
        n, d = x.shape
        qn, k, d2 = books.shape
        assert d == d2, "latent and codebook dims differ"
        q = qn if n_stages is None else int(n_stages)
        assert 0 < q <= qn
        assert np.isfinite(x).all() and np.isfinite(books).all(), "oracle inputs must be finite"
        codes = np.zeros((n, q), np.int32)
        residual = np.empty((n, d), np.float32)
        best = np.empty((n, q), np.float64)
        second = np.empty((n, q), np.float64)
        self.last_threads = self.lib.oracle_encode(
            x, n, d, books, q, k, codes, q, self._ptr(residual), self._ptr(best),
            self._ptr(second), int(threads))
        return codes, residual, best, second

    def decode(self, codes: np.ndarray, books: np.ndarray, threads: int = 0) -> np.ndarray:
        """Gather-sum decode: [N, Q] int32 codes -> [N, D] float32 (NaN frame on a bad code)."""
        codes = np.ascontiguousarray(codes, dtype=np.int32)
        books = np.ascontiguousarray(books, dtype=np.float32)
        n, q = codes.shape
        qn, k, d = books.shape
        assert q <= qn
        out = np.empty((n, d), np.float32)
        self.last_threads = self.lib.oracle_decode(codes, q, n, books, q, k, d, out, int(threads))
        return out

    def linear(self, h: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None,
               threads: int = 0) -> np.ndarray:
        """y = h W^T + b with W [out, in] (PyTorch order); float64 sums, float32 result."""
        h = np.ascontiguousarray(h, dtype=np.float32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        n, i = h.shape
        o, i2 = w.shape
        assert i == i2
        if b is not None:
            b = np.ascontiguousarray(b, dtype=np.float32)
            assert b.shape == (o,)
        y = np.empty((n, o), np.float32)
        self.last_threads = self.lib.oracle_linear(h, n, i, w, self._ptr(b), o, y, int(threads))
        return y

    @staticmethod
    def _projected_shapes(books, w_in, b_in, w_out, b_out, n_stages):
        books = np.ascontiguousarray(books, dtype=np.float32)
        qn, k, d = books.shape
        q = qn if n_stages is None else int(n_stages)
        assert 0 < q <= qn
        w_out = np.ascontiguousarray(w_out, dtype=np.float32)
        assert w_out.shape[0] >= q and w_out.shape[2] == d
        hidden = w_out.shape[1]
        if w_in is not None:
            w_in = np.ascontiguousarray(w_in, dtype=np.float32)
            assert w_in.shape[0] >= q and w_in.shape[1:] == (d, hidden)
        if b_in is not None:
            b_in = np.ascontiguousarray(b_in, dtype=np.float32)
            assert b_in.shape[0] >= q and b_in.shape[1] == d
        if b_out is not None:
            b_out = np.ascontiguousarray(b_out, dtype=np.float32)
            assert b_out.shape[0] >= q and b_out.shape[1] == hidden
        return books, w_in, b_in, w_out, b_out, q, k, d, hidden

    def projected_encode(self, h: np.ndarray, w_in: np.ndarray, b_in: Optional[np.ndarray],
                         books: np.ndarray, w_out: np.ndarray, b_out: Optional[np.ndarray],
                         n_stages: Optional[int] = None, e_given: Optional[np.ndarray] = None,
                         normalize: bool = False, threads: int = 0):
        """Per-stage projected encode (each codebook with its own project_in / project_out).

        ``h`` [N, hidden]; ``w_in`` [Q, D, hidden], ``b_in`` [Q, D] or None;
        ``books`` [Q, K, D]; ``w_out`` [Q, hidden, D], ``b_out`` [Q, hidden]
        or None. With ``e_given`` [Q, N, D] the argmin of stage q is taken on
        ``e_given[q]`` instead of the oracle's own projection. With
        ``normalize`` the argmin compares the encoding and the codewords
        scaled to unit L2 norm (float64, norm floored at 1e-12). Returns
        ``(codes [N, Q], e [Q, N, D] (the oracle's own projections),
        residual [N, hidden], best [N, Q], second [N, Q])``.
        """
        books, w_in, b_in, w_out, b_out, q, k, d, hidden = self._projected_shapes(
            books, w_in, b_in, w_out, b_out, n_stages)
        h = np.ascontiguousarray(h, dtype=np.float32)
        n = h.shape[0]
        assert h.shape[1] == hidden
        assert np.isfinite(h).all(), "oracle inputs must be finite"
        if e_given is not None:
            e_given = np.ascontiguousarray(e_given, dtype=np.float32)
            assert e_given.shape == (q, n, d)
        codes = np.zeros((n, q), np.int32)
        e = np.empty((q, n, d), np.float32)
        residual = np.empty((n, hidden), np.float32)
        best = np.empty((n, q), np.float64)
        second = np.empty((n, q), np.float64)
        self.last_threads = self.lib.oracle_projected_encode(
            h, n, hidden, w_in, self._ptr(b_in), books, q, k, d, w_out, self._ptr(b_out),
            self._ptr(e_given), codes, q, self._ptr(e), self._ptr(residual), self._ptr(best),
            self._ptr(second), int(bool(normalize)), int(threads))
        return codes, e, residual, best, second

    def projected_decode(self, codes: np.ndarray, books: np.ndarray, w_out: np.ndarray,
                         b_out: Optional[np.ndarray], threads: int = 0) -> np.ndarray:
        """Sum over stages of W_out[q] C[q, code] + b_out[q]: [N, Q] codes -> [N, hidden]."""
        codes = np.ascontiguousarray(codes, dtype=np.int32)
        n, q = codes.shape
        books, _, _, w_out, b_out, q, k, d, hidden = self._projected_shapes(
            books, None, None, w_out, b_out, q)
        out = np.empty((n, hidden), np.float32)
        self.last_threads = self.lib.oracle_projected_decode(
            codes, q, n, books, q, k, d, w_out, self._ptr(b_out), hidden, out, int(threads))
        return out

    def roundtrip(self, x: np.ndarray, books: np.ndarray, threads: int = 0):
        """Encode then decode: returns ``(codes, recon, residual, best, second)``."""
        codes, residual, best, second = self.encode(x, books, threads=threads)
        recon = self.decode(codes, books, threads=threads)
        return codes, recon, residual, best, second


def near_tie(best: np.ndarray, second: np.ndarray, rel: float = 1e-5) -> np.ndarray:
    """Stage-wise near-tie flag: second - best <= rel * best (no division, so 0 == 0 ties)."""
    return (second - best) <= rel * best


_default: Optional[Oracle] = None


def get(rebuild: bool = False) -> Oracle:
    """The default oracle build, compiling it first if it is missing or stale."""
    global _default
    if _default is None or rebuild:
        stale = (not os.path.exists(LIBRARY)
                 or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE))
        if rebuild or stale:
            build()
        _default = Oracle(LIBRARY)
    return _default
