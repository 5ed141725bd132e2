"""Residual vector quantization on MI355X (gfx950): Python binding of librvq.

Thin ctypes layer over the C ABI in ``include/rvq.h``. It checks tensor
dtypes, devices and layouts, allocates outputs with ``torch.empty`` on the
input's device, and passes raw device pointers plus the current HIP stream.
Every step of encode and decode runs in the HIP kernels of ``librvq.so``;
there is no CPU or PyTorch fallback. If the library is missing the import
still works, but every call raises.

Functions (same names as the C entry points):

* ``rvq_encode(x, codebooks, n_stages=None, residual=True)``
  -> ``(codes [N, Q] int32, residual [N, D] float32 or None)``
* ``rvq_decode(codes, codebooks, n_stages=None)`` -> ``out [N, D] float32``
* ``rvq_roundtrip(x, codebooks, n_stages=None, residual=True)``
  -> ``(codes, recon, residual or None)``
* ``rvq_encode_scored(x, codebooks, scoring, n_stages=None, recon=True, residual=True)``
  -> ``(codes, recon or None, residual or None)``; scoring "default", "bf16x3" or "fp32"
* ``rvq_prepared_bytes(n_stages, n_codes, dim)`` -> int;
  ``rvq_prepare_codebooks(codebooks)`` -> uint8 device tensor;
  ``rvq_encode_prepared(x, codebooks, prepared, n_stages=None, recon=False, residual=True)``
  -> ``(codes, recon or None, residual or None)``
* ``rvq_encode_noalloc(x, codebooks, n_stages=None, recon=False, residual=True)``
  -> ``(codes, recon or None, residual or None)``: the prepared encode with the library's own fixed
  per-GPU buffer, allocating nothing in the C call
* ``rvq_project_roundtrip(h, w_in, b_in, codebooks, w_out, b_out, n_stages=None, prepared=None)``
  -> ``(codes, latent, latent_recon, h_recon)``
* ``rvq_projected_prepare(codebooks, w_out, b_out=None)`` -> table;
  ``rvq_projected_encode(h, w_in, b_in, codebooks, table, n_stages=None, prepared=None)``
  -> ``(codes, latent, residual)``; ``rvq_projected_decode(codes, table, n_stages=None)``
* ``rvq_cosine_prepare(codebooks)`` -> unit codewords (float64);
  ``rvq_cosine_encode(h, w_in, b_in, units, table, n_stages=None)`` -> ``(codes, latent, residual)``
* ``rvq_version()``, ``rvq_status_string(status)``

``prepared`` is ``rvq_prepare_codebooks``' output for the same codebooks; passing it selects
the encode that reads the prepared layout (same results, faster).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "librvq.so")

RVQ_OK = 0
RVQ_ERR_INVALID_ARG = -1
RVQ_ERR_UNSUPPORTED = -2
RVQ_ERR_DEVICE = -3
RVQ_ERR_OOM = -4

EXPORTED = ("rvq_version", "rvq_status_string", "rvq_encode", "rvq_decode", "rvq_roundtrip",
            "rvq_encode_scored", "rvq_prepared_bytes", "rvq_prepare_codebooks", "rvq_encode_prepared",
            "rvq_project_roundtrip", "rvq_projected_prepare", "rvq_projected_encode", "rvq_projected_decode",
            "rvq_cosine_prepare", "rvq_cosine_encode", "rvq_encode_noalloc")

# Bytes of the library's per-GPU array behind rvq_encode_noalloc (RVQ_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024

SCORING = {"default": 0, "bf16x3": 1, "fp32": 2}

_lib = None


class RVQError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {message} ({status})")
        self.status = status


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Loads librvq.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing; build it with `python -m residual_vector_quantization_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.rvq_version.restype = ctypes.c_char_p
    lib.rvq_version.argtypes = []
    lib.rvq_status_string.restype = ctypes.c_char_p
    lib.rvq_status_string.argtypes = [ctypes.c_int]
    lib.rvq_encode.restype = ctypes.c_int
    lib.rvq_encode.argtypes = [vp, i64, i32, vp, i32, i32, vp, i32, vp, vp]
    lib.rvq_decode.restype = ctypes.c_int
    lib.rvq_decode.argtypes = [vp, i32, i64, vp, i32, i32, i32, vp, vp]
    lib.rvq_roundtrip.restype = ctypes.c_int
    lib.rvq_roundtrip.argtypes = [vp, i64, i32, vp, i32, i32, vp, i32, vp, vp, vp]
    lib.rvq_encode_scored.restype = ctypes.c_int
    lib.rvq_encode_scored.argtypes = [vp, i64, i32, vp, i32, i32, vp, i32, vp, vp, ctypes.c_int, vp]
    lib.rvq_prepared_bytes.restype = ctypes.c_int64
    lib.rvq_prepared_bytes.argtypes = [i32, i32, i32]
    lib.rvq_prepare_codebooks.restype = ctypes.c_int
    lib.rvq_prepare_codebooks.argtypes = [vp, i32, i32, i32, vp, i64, vp]
    lib.rvq_encode_prepared.restype = ctypes.c_int
    lib.rvq_encode_prepared.argtypes = [vp, i64, i32, vp, vp, i32, i32, vp, i32, vp, vp, vp]
    lib.rvq_project_roundtrip.restype = ctypes.c_int
    lib.rvq_project_roundtrip.argtypes = [vp, i64, i32, vp, vp, vp, vp, i32, i32, i32, vp, vp,
                                          vp, i32, vp, vp, vp, vp]
    lib.rvq_projected_prepare.restype = ctypes.c_int
    lib.rvq_projected_prepare.argtypes = [vp, i32, i32, i32, vp, vp, i32, vp, vp]
    lib.rvq_projected_encode.restype = ctypes.c_int
    lib.rvq_projected_encode.argtypes = [vp, i64, i32, vp, vp, vp, vp, vp, i32, i32, i32, vp, i32, vp, vp, vp]
    lib.rvq_projected_decode.restype = ctypes.c_int
    lib.rvq_projected_decode.argtypes = [vp, i32, i64, vp, i32, i32, i32, vp, vp]
    lib.rvq_cosine_prepare.restype = ctypes.c_int
    lib.rvq_cosine_prepare.argtypes = [vp, i32, i32, i32, vp, vp]
    lib.rvq_encode_noalloc.restype = ctypes.c_int
    lib.rvq_encode_noalloc.argtypes = [vp, i64, i32, vp, i32, i32, vp, i32, vp, vp, vp]
    lib.rvq_cosine_encode.restype = ctypes.c_int
    lib.rvq_cosine_encode.argtypes = [vp, i64, i32, vp, vp, vp, vp, i32, i32, i32, vp, i32, vp, vp, vp]
    _lib = lib
    return lib


def rvq_version() -> str:
    return load().rvq_version().decode()


def rvq_status_string(status: int) -> str:
    return load().rvq_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != RVQ_OK:
        raise RVQError(fn, status, rvq_status_string(status))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t: torch.Tensor, name: str, dtype: torch.dtype, dims: int, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stages(codebooks: torch.Tensor, n_stages: Optional[int]) -> int:
    q = codebooks.shape[0] if n_stages is None else int(n_stages)
    if not 0 < q <= codebooks.shape[0]:
        raise ValueError(f"n_stages={q} outside 1..{codebooks.shape[0]}")
    return q


def _check_dims(x: torch.Tensor, codebooks: torch.Tensor) -> None:
    """The C ABI takes the latent width from ``x`` alone, so the codebooks' rows must have it too."""
    if codebooks.shape[2] != x.shape[1]:
        raise ValueError(f"codebooks {tuple(codebooks.shape)} do not match x {tuple(x.shape)} in the last dim")


def _check_codes(codes: torch.Tensor, n: int, q: int) -> None:
    """An output codes tensor needs one row per frame and at least ``q`` columns."""
    if codes.shape[0] != n:
        raise ValueError(f"codes must have one row per frame ({n}), got {tuple(codes.shape)}")
    if codes.shape[1] < q:
        raise ValueError(f"codes needs at least {q} columns, got {tuple(codes.shape)}")


def rvq_encode(x: torch.Tensor, codebooks: torch.Tensor, n_stages: Optional[int] = None,
               residual: bool = True, codes: Optional[torch.Tensor] = None,
               residual_out: Optional[torch.Tensor] = None):
    """Greedy residual encode of ``x`` [N, D] against ``codebooks`` [Q, K, D].

    Returns ``(codes [N, Q] int32, residual [N, D] float32 or None)``. ``codes``
    may be a preallocated [N, L] int32 tensor with L >= Q (columns 0..Q-1 are
    written); ``residual_out`` a preallocated [N, D] float32 tensor.
    """
    _require(x, "x", torch.float32, 2)
    _require(codebooks, "codebooks", torch.float32, 3, x.device)
    _check_dims(x, codebooks)
    n, d = x.shape
    q = _stages(codebooks, n_stages)
    if codes is None:
        codes = torch.empty((n, q), dtype=torch.int32, device=x.device)
    _require(codes, "codes", torch.int32, 2, x.device)
    _check_codes(codes, n, q)
    res = None
    if residual:
        res = residual_out if residual_out is not None else torch.empty_like(x)
        _require(res, "residual", torch.float32, 2, x.device)
        if res.shape != x.shape:
            raise ValueError("residual must match x")
    st = load().rvq_encode(_ptr(x), n, d, _ptr(codebooks), q, codebooks.shape[1],
                           _ptr(codes), codes.shape[1], _ptr(res), _stream(x))
    _check("rvq_encode", st)
    return codes, res


def rvq_decode(codes: torch.Tensor, codebooks: torch.Tensor, n_stages: Optional[int] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gather-sum decode: ``codes`` [N, L] int32 (first Q columns) -> [N, D] float32."""
    _require(codes, "codes", torch.int32, 2)
    _require(codebooks, "codebooks", torch.float32, 3, codes.device)
    n = codes.shape[0]
    q = codes.shape[1] if n_stages is None else int(n_stages)
    if not 0 < q <= min(codes.shape[1], codebooks.shape[0]):
        raise ValueError(f"n_stages={q} does not fit codes {tuple(codes.shape)} / codebooks")
    d = codebooks.shape[2]
    if out is None:
        out = torch.empty((n, d), dtype=torch.float32, device=codes.device)
    _require(out, "out", torch.float32, 2, codes.device)
    if out.shape != (n, d):
        raise ValueError("out must be [N, D]")
    st = load().rvq_decode(_ptr(codes), codes.shape[1], n, _ptr(codebooks), q, codebooks.shape[1],
                           d, _ptr(out), _stream(codes))
    _check("rvq_decode", st)
    return out


def rvq_roundtrip(x: torch.Tensor, codebooks: torch.Tensor, n_stages: Optional[int] = None,
                  residual: bool = True):
    """Encode and reconstruct in one pass: ``(codes, recon, residual or None)``.

    ``recon`` equals ``rvq_decode(codes, codebooks)`` bit for bit.
    """
    _require(x, "x", torch.float32, 2)
    _require(codebooks, "codebooks", torch.float32, 3, x.device)
    _check_dims(x, codebooks)
    n, d = x.shape
    q = _stages(codebooks, n_stages)
    codes = torch.empty((n, q), dtype=torch.int32, device=x.device)
    recon = torch.empty_like(x)
    res = torch.empty_like(x) if residual else None
    st = load().rvq_roundtrip(_ptr(x), n, d, _ptr(codebooks), q, codebooks.shape[1],
                              _ptr(codes), q, _ptr(recon), _ptr(res), _stream(x))
    _check("rvq_roundtrip", st)
    return codes, recon, res


def rvq_encode_scored(x: torch.Tensor, codebooks: torch.Tensor, scoring: str = "default",
                      n_stages: Optional[int] = None, recon: bool = True, residual: bool = True,
                      out=None):
    """Encode with an explicit scoring ("default", "bf16x3" or "fp32"); all give identical results.

    Returns ``(codes, recon or None, residual or None)``; ``out`` may pass
    ``(codes, recon, residual)`` preallocated (entries may be None).
    """
    _require(x, "x", torch.float32, 2)
    _require(codebooks, "codebooks", torch.float32, 3, x.device)
    if scoring not in SCORING:
        raise ValueError(f"scoring must be one of {sorted(SCORING)}")
    _check_dims(x, codebooks)
    n, d = x.shape
    q = _stages(codebooks, n_stages)
    if out is None:
        out = (torch.empty((n, q), dtype=torch.int32, device=x.device),
               torch.empty_like(x) if recon else None, torch.empty_like(x) if residual else None)
    codes, rec, res = out
    _require(codes, "codes", torch.int32, 2, x.device)
    _check_codes(codes, n, q)
    for t, name in ((rec, "recon"), (res, "residual")):
        if t is not None:
            _require(t, name, torch.float32, 2, x.device)
            if t.shape != x.shape:
                raise ValueError(f"{name} must match x")
    st = load().rvq_encode_scored(_ptr(x), n, d, _ptr(codebooks), q, codebooks.shape[1], _ptr(codes),
                                  codes.shape[1], _ptr(rec), _ptr(res), SCORING[scoring], _stream(x))
    _check("rvq_encode_scored", st)
    return codes, rec, res


def rvq_prepared_bytes(n_stages: int, n_codes: int, dim: int) -> int:
    size = load().rvq_prepared_bytes(n_stages, n_codes, dim)
    if size < 0:
        raise RVQError("rvq_prepared_bytes", size, rvq_status_string(size))
    return size


def rvq_prepare_codebooks(codebooks: torch.Tensor, prepared: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Prepared layout (per stage a power-of-two scale, fp16 rows and half-norm parts) of ``codebooks``
    [Q, K, D], as a uint8 tensor on the same device."""
    _require(codebooks, "codebooks", torch.float32, 3)
    q, k, d = codebooks.shape
    size = rvq_prepared_bytes(q, k, d)
    if prepared is None:
        prepared = torch.empty(size, dtype=torch.uint8, device=codebooks.device)
    _require(prepared, "prepared", torch.uint8, 1, codebooks.device)
    st = load().rvq_prepare_codebooks(_ptr(codebooks), q, k, d, _ptr(prepared), prepared.numel(),
                                      _stream(codebooks))
    _check("rvq_prepare_codebooks", st)
    return prepared


def _check_prepared(prepared: Optional[torch.Tensor], codebooks: torch.Tensor, q: int) -> None:
    """A prepared-codebook buffer, if given, must be a uint8 tensor on the codebooks' device large enough
    for their first ``q`` stages."""
    if prepared is None:
        return
    _require(prepared, "prepared", torch.uint8, 1, codebooks.device)
    if prepared.numel() < rvq_prepared_bytes(q, codebooks.shape[1], codebooks.shape[2]):
        raise ValueError("prepared buffer is too small for these codebooks")


def rvq_encode_prepared(x: torch.Tensor, codebooks: torch.Tensor, prepared: torch.Tensor,
                        n_stages: Optional[int] = None, recon: bool = False, residual: bool = True,
                        out=None):
    """Encode from prepared codebooks (fp16 scores, exact re-rank):
    ``(codes, recon or None, residual or None)``."""
    _require(x, "x", torch.float32, 2)
    _require(codebooks, "codebooks", torch.float32, 3, x.device)
    _require(prepared, "prepared", torch.uint8, 1, x.device)
    _check_dims(x, codebooks)
    n, d = x.shape
    q = _stages(codebooks, n_stages)
    if prepared.numel() < rvq_prepared_bytes(q, codebooks.shape[1], d):
        raise ValueError("prepared buffer is too small for these codebooks")
    if out is None:
        out = (torch.empty((n, q), dtype=torch.int32, device=x.device),
               torch.empty_like(x) if recon else None, torch.empty_like(x) if residual else None)
    codes, rec, res = out
    _require(codes, "codes", torch.int32, 2, x.device)
    _check_codes(codes, n, q)
    for t, name in ((rec, "recon"), (res, "residual")):
        if t is not None:
            _require(t, name, torch.float32, 2, x.device)
            if t.shape != x.shape:
                raise ValueError(f"{name} must match x")
    st = load().rvq_encode_prepared(_ptr(x), n, d, _ptr(codebooks), _ptr(prepared), q, codebooks.shape[1],
                                    _ptr(codes), codes.shape[1], _ptr(rec), _ptr(res), _stream(x))
    _check("rvq_encode_prepared", st)
    return codes, rec, res


def rvq_encode_noalloc(x: torch.Tensor, codebooks: torch.Tensor, n_stages: Optional[int] = None,
                       recon: bool = False, residual: bool = True, out=None):
    """``rvq_encode_prepared`` with the prepared layout in the library's fixed per-GPU array
    (``NOALLOC_SCRATCH_BYTES``) instead of a caller buffer; the C call allocates nothing. Pass ``out``
    = ``(codes, recon or None, residual or None)`` preallocated to keep the whole call allocation-free.
    Calls that overlap on one GPU race on the array. Returns ``(codes, recon or None, residual or None)``."""
    _require(x, "x", torch.float32, 2)
    _require(codebooks, "codebooks", torch.float32, 3, x.device)
    _check_dims(x, codebooks)
    n, d = x.shape
    q = _stages(codebooks, n_stages)
    if out is None:
        out = (torch.empty((n, q), dtype=torch.int32, device=x.device),
               torch.empty_like(x) if recon else None, torch.empty_like(x) if residual else None)
    codes, rec, res = out
    _require(codes, "codes", torch.int32, 2, x.device)
    _check_codes(codes, n, q)
    for t, name in ((rec, "recon"), (res, "residual")):
        if t is not None:
            _require(t, name, torch.float32, 2, x.device)
            if t.shape != x.shape:
                raise ValueError(f"{name} must match x")
    st = load().rvq_encode_noalloc(_ptr(x), n, d, _ptr(codebooks), q, codebooks.shape[1], _ptr(codes),
                                   codes.shape[1], _ptr(rec), _ptr(res), _stream(x))
    _check("rvq_encode_noalloc", st)
    return codes, rec, res


def rvq_project_roundtrip(h: torch.Tensor, w_in: torch.Tensor, b_in: Optional[torch.Tensor],
                          codebooks: torch.Tensor, w_out: torch.Tensor, b_out: Optional[torch.Tensor],
                          n_stages: Optional[int] = None, out=None, prepared: Optional[torch.Tensor] = None):
    """fc -> encode -> decode -> fc2 on ``h`` [N, H].

    ``w_in`` [D, H], ``w_out`` [H, D] in PyTorch (out, in) order, biases
    [D] / [H] or None. Returns ``(codes [N, Q], latent [N, D],
    latent_recon [N, D], h_recon [N, H])``; ``out`` may pass those four
    tensors preallocated. ``prepared``: optional ``rvq_prepare_codebooks``
    output for ``codebooks`` (same results, faster encode).
    """
    _require(h, "h", torch.float32, 2)
    dev = h.device
    _require(codebooks, "codebooks", torch.float32, 3, dev)
    _require(w_in, "w_in", torch.float32, 2, dev)
    _require(w_out, "w_out", torch.float32, 2, dev)
    n, hid = h.shape
    d = codebooks.shape[2]
    if tuple(w_in.shape) != (d, hid) or tuple(w_out.shape) != (hid, d):
        raise ValueError("w_in must be [D, H] and w_out [H, D]")
    for b, name, size in ((b_in, "b_in", d), (b_out, "b_out", hid)):
        if b is not None:
            _require(b, name, torch.float32, 1, dev)
            if b.shape[0] != size:
                raise ValueError(f"{name} must have {size} entries")
    q = _stages(codebooks, n_stages)
    _check_prepared(prepared, codebooks, q)
    if out is None:
        out = (torch.empty((n, q), dtype=torch.int32, device=dev),
               torch.empty((n, d), dtype=torch.float32, device=dev),
               torch.empty((n, d), dtype=torch.float32, device=dev),
               torch.empty((n, hid), dtype=torch.float32, device=dev))
    codes, latent, latent_recon, h_recon = out
    _require(codes, "codes", torch.int32, 2, dev)
    _check_codes(codes, n, q)
    for t, name, width in ((latent, "latent", d), (latent_recon, "latent_recon", d), (h_recon, "h_recon", hid)):
        _require(t, name, torch.float32, 2, dev)
        if tuple(t.shape) != (n, width):
            raise ValueError(f"{name} must be [{n}, {width}], got {tuple(t.shape)}")
    st = load().rvq_project_roundtrip(_ptr(h), n, hid, _ptr(w_in), _ptr(b_in), _ptr(codebooks), _ptr(prepared),
                                      q, codebooks.shape[1], d, _ptr(w_out), _ptr(b_out), _ptr(codes),
                                      codes.shape[1], _ptr(latent), _ptr(latent_recon), _ptr(h_recon),
                                      _stream(h))
    _check("rvq_project_roundtrip", st)
    return codes, latent, latent_recon, h_recon


def rvq_projected_prepare(codebooks: torch.Tensor, w_out: torch.Tensor, b_out: Optional[torch.Tensor] = None,
                          table: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Table of projected codewords ``[Q, K, H]``: ``W_out[q] C[q, k] + b_out[q]``.

    ``codebooks`` [Q, K, D], ``w_out`` [Q, H, D] (PyTorch (out, in) order per
    stage), ``b_out`` [Q, H] or None.
    """
    _require(codebooks, "codebooks", torch.float32, 3)
    dev = codebooks.device
    _require(w_out, "w_out", torch.float32, 3, dev)
    q, k, d = codebooks.shape
    if w_out.shape[0] != q or w_out.shape[2] != d:
        raise ValueError("w_out must be [Q, H, D] (D = 64, or 8 for the normalized quantizer)")
    hid = w_out.shape[1]
    if b_out is not None:
        _require(b_out, "b_out", torch.float32, 2, dev)
        if tuple(b_out.shape) != (q, hid):
            raise ValueError("b_out must be [Q, H]")
    if table is None:
        table = torch.empty((q, k, hid), dtype=torch.float32, device=dev)
    _require(table, "table", torch.float32, 3, dev)
    if tuple(table.shape) != (q, k, hid):
        raise ValueError("table must be [Q, K, H]")
    st = load().rvq_projected_prepare(_ptr(codebooks), q, k, d, _ptr(w_out), _ptr(b_out), hid, _ptr(table),
                                      _stream(codebooks))
    _check("rvq_projected_prepare", st)
    return table


def rvq_projected_encode(h: torch.Tensor, w_in: torch.Tensor, b_in: Optional[torch.Tensor],
                         codebooks: torch.Tensor, table: torch.Tensor, n_stages: Optional[int] = None,
                         out=None, prepared: Optional[torch.Tensor] = None):
    """Per-stage projected encode of ``h`` [N, H].

    ``w_in`` [Q, D, H], ``b_in`` [Q, D] or None, ``table`` from
    ``rvq_projected_prepare``. Returns ``(codes [N, Q], latent [Q, N, D],
    residual [N, H])``; ``out`` may pass those three tensors preallocated
    (codes may be [N, L] with L >= Q). ``prepared``: optional
    ``rvq_prepare_codebooks`` output for ``codebooks`` (same results,
    faster argmin).
    """
    _require(h, "h", torch.float32, 2)
    dev = h.device
    _require(codebooks, "codebooks", torch.float32, 3, dev)
    _require(w_in, "w_in", torch.float32, 3, dev)
    _require(table, "table", torch.float32, 3, dev)
    n, hid = h.shape
    qn, k, d = codebooks.shape
    q = _stages(codebooks, n_stages)
    if w_in.shape[0] < q or tuple(w_in.shape[1:]) != (d, hid):
        raise ValueError("w_in must be [Q, D, H]")
    if b_in is not None:
        _require(b_in, "b_in", torch.float32, 2, dev)
        if b_in.shape[0] < q or b_in.shape[1] != d:
            raise ValueError("b_in must be [Q, D]")
    if table.shape[0] < q or tuple(table.shape[1:]) != (k, hid):
        raise ValueError("table must be [Q, K, H]")
    if out is None:
        out = (torch.empty((n, q), dtype=torch.int32, device=dev),
               torch.empty((q, n, d), dtype=torch.float32, device=dev),
               torch.empty((n, hid), dtype=torch.float32, device=dev))
    codes, latent, residual = out
    _require(codes, "codes", torch.int32, 2, dev)
    _require(latent, "latent", torch.float32, 3, dev)
    _require(residual, "residual", torch.float32, 2, dev)
    if codes.shape[0] != n or codes.shape[1] < q or latent.shape[0] < q or tuple(latent.shape[1:]) != (n, d) \
            or residual.shape != h.shape:
        raise ValueError("output shapes do not match")
    _check_prepared(prepared, codebooks, q)
    st = load().rvq_projected_encode(_ptr(h), n, hid, _ptr(w_in), _ptr(b_in), _ptr(codebooks), _ptr(prepared),
                                     _ptr(table), q, k, d, _ptr(codes), codes.shape[1], _ptr(latent),
                                     _ptr(residual), _stream(h))
    _check("rvq_projected_encode", st)
    return codes, latent, residual


def rvq_projected_decode(codes: torch.Tensor, table: torch.Tensor, n_stages: Optional[int] = None,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sum of projected codewords: ``codes`` [N, L] (first Q columns) -> [N, H]."""
    _require(codes, "codes", torch.int32, 2)
    _require(table, "table", torch.float32, 3, codes.device)
    n = codes.shape[0]
    q = table.shape[0] if n_stages is None else int(n_stages)
    if not 0 < q <= min(codes.shape[1], table.shape[0]):
        raise ValueError(f"n_stages={q} does not fit codes {tuple(codes.shape)} / table")
    k, hid = table.shape[1], table.shape[2]
    if out is None:
        out = torch.empty((n, hid), dtype=torch.float32, device=codes.device)
    _require(out, "out", torch.float32, 2, codes.device)
    if tuple(out.shape) != (n, hid):
        raise ValueError("out must be [N, H]")
    st = load().rvq_projected_decode(_ptr(codes), codes.shape[1], n, _ptr(table), q, k, hid, _ptr(out),
                                     _stream(codes))
    _check("rvq_projected_decode", st)
    return out


def rvq_cosine_prepare(codebooks: torch.Tensor, units: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Unit codewords ``[Q, K, 8]`` float64 of 8-dim ``codebooks`` [Q, K, 8] (norm floor 1e-12)."""
    _require(codebooks, "codebooks", torch.float32, 3)
    q, k, d = codebooks.shape
    if units is None:
        units = torch.empty((q, k, d), dtype=torch.float64, device=codebooks.device)
    _require(units, "units", torch.float64, 3, codebooks.device)
    if tuple(units.shape) != (q, k, d):
        raise ValueError("units must be [Q, K, D]")
    st = load().rvq_cosine_prepare(_ptr(codebooks), q, k, d, _ptr(units), _stream(codebooks))
    _check("rvq_cosine_prepare", st)
    return units


def rvq_cosine_encode(h: torch.Tensor, w_in: torch.Tensor, b_in: Optional[torch.Tensor], units: torch.Tensor,
                      table: torch.Tensor, n_stages: Optional[int] = None, out=None):
    """Normalized (cosine) per-stage projected encode of ``h`` [N, H].

    ``w_in`` [Q, 8, H], ``b_in`` [Q, 8] or None, ``units`` from
    ``rvq_cosine_prepare``, ``table`` from ``rvq_projected_prepare`` (8-dim
    codebooks). Returns ``(codes [N, Q], latent [Q, N, 8], residual [N, H])``;
    ``out`` may pass those three tensors preallocated.
    """
    _require(h, "h", torch.float32, 2)
    dev = h.device
    _require(w_in, "w_in", torch.float32, 3, dev)
    _require(units, "units", torch.float64, 3, dev)
    _require(table, "table", torch.float32, 3, dev)
    n, hid = h.shape
    qn, k, d = units.shape
    q = qn if n_stages is None else int(n_stages)
    if not 0 < q <= qn:
        raise ValueError(f"n_stages={q} outside 1..{qn}")
    if w_in.shape[0] < q or tuple(w_in.shape[1:]) != (d, hid):
        raise ValueError("w_in must be [Q, D, H]")
    if b_in is not None:
        _require(b_in, "b_in", torch.float32, 2, dev)
        if b_in.shape[0] < q or b_in.shape[1] != d:
            raise ValueError("b_in must be [Q, D]")
    if table.shape[0] < q or tuple(table.shape[1:]) != (k, hid):
        raise ValueError("table must be [Q, K, H]")
    if out is None:
        out = (torch.empty((n, q), dtype=torch.int32, device=dev),
               torch.empty((q, n, d), dtype=torch.float32, device=dev),
               torch.empty((n, hid), dtype=torch.float32, device=dev))
    codes, latent, residual = out
    _require(codes, "codes", torch.int32, 2, dev)
    _require(latent, "latent", torch.float32, 3, dev)
    _require(residual, "residual", torch.float32, 2, dev)
    if codes.shape[0] != n or codes.shape[1] < q or latent.shape[0] < q or tuple(latent.shape[1:]) != (n, d) \
            or residual.shape != h.shape:
        raise ValueError("output shapes do not match")
    st = load().rvq_cosine_encode(_ptr(h), n, hid, _ptr(w_in), _ptr(b_in), _ptr(units), _ptr(table), q, k, d,
                                  _ptr(codes), codes.shape[1], _ptr(latent), _ptr(residual), _stream(h))
    _check("rvq_cosine_encode", st)
    return codes, latent, residual
