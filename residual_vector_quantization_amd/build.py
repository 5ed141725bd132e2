"""Builds librvq.so (HIP, gfx950 only) in-tree.

    python -m residual_vector_quantization_amd.build

Every call recompiles; the objects go to ``_build/`` next to this file and
the shared library to ``librvq.so`` inside the package.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "librvq.so")
# measurement tooling beside the library: the ceilings (row gathers, matrix cores) the kernels are compared with
PROBE_LIBRARY = os.path.join(PKG, "librvq_probe.so")
PROBE_SOURCES = ["probes.hip"]
SOURCES = ["rvq_api.hip", "encode.hip", "encode_bf16.hip", "encode_f16.hip", "decode.hip", "linear.hip", "projected.hip",
           "cosine.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # float64 re-rank sums and float32 residual/decode sums must round per operation
    "-ffp-contract=off",
    # no packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    subprocess.run([HIPCC, *CXXFLAGS, "-c", os.path.join(CSRC, src), "-o", obj], check=True)
    return obj


def _link(objs, target):
    tmp = target + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, target)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(PROBE_SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIBRARY)
    _link(objs[len(SOURCES):], PROBE_LIBRARY)
    if verbose:
        print("built", LIBRARY, PROBE_LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
