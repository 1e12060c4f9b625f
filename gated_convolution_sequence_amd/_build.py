"""Build step for the HIP library (hipcc, gfx950, in-tree)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", name) for name in ("hyena_conv.hip", "hyena_fft.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhyena_conv.so")
# the benchmark's streaming reference kernel (not part of the operator's ABI)
STREAM_REF_SOURCE = os.path.join(PKG, "csrc", "stream_ref.hip")
STREAM_REF_LIB = os.path.join(PKG, "libhyena_stream_ref.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(sources, lib, verbose):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I" + INCLUDE, "-o", tmp, *sources]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, lib)
    return lib


def build_library(verbose: bool = False) -> str:
    """Compile the operator's csrc/*.hip sources into libhyena_conv.so next to this file."""
    return _compile(SOURCES, LIB, verbose)


def build_stream_ref(verbose: bool = False) -> str:
    """Compile the benchmark's streaming reference kernel into libhyena_stream_ref.so."""
    return _compile([STREAM_REF_SOURCE], STREAM_REF_LIB, verbose)
