"""The C ABI library loads, exports what include/rvq.h declares, and rejects bad arguments (no GPU)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rvq.h")


@pytest.fixture(scope="module")
def libpath():
    from residual_vector_quantization_amd import build, LIBRARY
    if not os.path.exists(LIBRARY):
        build.build()
    return LIBRARY


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"RVQ_API[^;(]*?\b(rvq_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared() == sorted(["rvq_cosine_encode", "rvq_cosine_prepare",
                                 "rvq_decode", "rvq_encode", "rvq_encode_noalloc", "rvq_encode_prepared",
                                 "rvq_encode_scored",
                                 "rvq_prepare_codebooks", "rvq_prepared_bytes", "rvq_project_roundtrip",
                                 "rvq_projected_decode", "rvq_projected_encode", "rvq_projected_prepare",
                                 "rvq_roundtrip", "rvq_status_string", "rvq_version"])


def test_library_exports_every_declared_symbol(libpath):
    lib = ctypes.CDLL(libpath)
    for name in declared():
        assert hasattr(lib, name), name


def test_only_rvq_symbols_exported(libpath):
    out = subprocess.run(["nm", "-D", "--defined-only", libpath], capture_output=True, text=True,
                         check=True).stdout
    names = [ln.split()[-1] for ln in out.splitlines() if ln.strip() and ln.split()[-2] in "TtWw"]
    own = [n for n in names if not n.startswith("_")]
    assert own and all(n.startswith("rvq_") for n in own), own


def test_binding_names_match_header():
    import residual_vector_quantization_amd as rvq
    assert sorted(rvq.EXPORTED) == declared()
    for name in declared():
        assert callable(getattr(rvq, name))


def test_c99_consumer_compiles_and_validates(tmp_path, libpath):
    exe = tmp_path / "abi_c99"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "abi_c99.c"), libpath, "-o", str(exe),
                    "-Wl,-rpath," + os.path.dirname(libpath)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_c99: ok" in r.stdout


def test_status_strings(libpath):
    import residual_vector_quantization_amd as rvq
    assert rvq.rvq_status_string(0) == "ok"
    assert rvq.rvq_status_string(-2) == "unsupported shape"
    assert rvq.rvq_status_string(-4) == "out of memory"
    assert rvq.rvq_status_string(-99) == "unknown status"
    assert "gfx950" in rvq.rvq_version()


def test_prepared_bytes_shape_rules(libpath):
    import residual_vector_quantization_amd as rvq
    a = rvq.rvq_prepared_bytes(8, 1024, 64)
    # per stage: 144-byte rows, one maximum per 256 rows and the scale, in a 256-byte aligned block
    assert a == 8 * ((1024 * 144 + 4 * 4 + 4 + 255) // 256 * 256)
    assert rvq.rvq_prepared_bytes(8, 1000, 64) == a   # rows are padded to whole chunks
    assert rvq.rvq_prepared_bytes(1, 1, 64) > 0
    with pytest.raises(rvq.RVQError):
        rvq.rvq_prepared_bytes(8, 1024, 32)
