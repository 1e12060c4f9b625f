"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The C ABI does all of its argument checking, planning and alias tests on
the host before any HIP call.  This test rebuilds the library with the
sanitizers on the host side only (hipcc -Xarch_host before every sanitizer
flag; device code is built as usual) into a temporary directory, and runs
the whole host ABI suite (tests/test_abi.py) against it in a child process
that preloads the clang ASan runtime.  Any out-of-bounds access or undefined
operation on the host aborts the child; the sanitizer reports are written
to files and shown on failure.  About a minute, most of it the device build.
"""
import glob
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "gated_convolution_sequence_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

CHILD = textwrap.dedent('''
    import sys
    sys.path.insert(0, sys.argv[2]); sys.path.insert(0, sys.argv[2] + "/tests")
    import gated_convolution_sequence_amd as hc
    hc.LIB_PATH = sys.argv[1]            # the sanitized build
    import pytest
    sys.exit(pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                          sys.argv[2] + "/tests/test_abi.py"]))
''')


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_host_code_clean_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not installed")
    lib = str(tmp_path / "libhyena_conv_san.so")
    san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer", "-shared-libsan"):
        san += ["-Xarch_host", flag]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include")]
    cmd += san + ["-o", lib, os.path.join(CSRC, "hyena_conv.hip"), os.path.join(CSRC, "hyena_fft.hip")]
    subprocess.run(cmd, check=True, capture_output=True)
    logs = str(tmp_path / "san")
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:log_path=" + logs,
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:log_path=" + logs)
    r = subprocess.run([sys.executable, "-c", CHILD, lib, ROOT], env=env, capture_output=True, text=True,
                       timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(logs + "*"))
    assert r.returncode == 0 and not reports, reports[-4000:] + r.stdout[-2000:] + r.stderr[-2000:]
    assert "passed" in r.stdout, r.stdout[-2000:]
