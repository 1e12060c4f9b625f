"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host, CPU).

The C oracle is rebuilt with gcc -fsanitize=address,undefined into a
temporary directory and driven from a child process that preloads the ASan
runtime, on small shapes that reach every boundary of its loops (L = 1,
l_h > L, l_h = 1, several batch rows, group sizes 1 to D).  Any out-of-bounds
access or undefined operation aborts the child; its results must also equal
a direct NumPy evaluation of the definition, forward and backward.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "hyena_ref.c")

CHILD = textwrap.dedent('''
    import sys
    import numpy as np
    sys.path.insert(0, sys.argv[2])
    import oracle
    oracle._LIB = sys.argv[1]            # the sanitized build
    rng = np.random.default_rng(7)

    def direct(q, k, v, h, gs):
        B, L, D = q.shape
        x = k * v
        y = np.zeros_like(q)
        for d in range(D):
            hd = h[d // gs]
            for t in range(L):
                s = min(t, hd.shape[0] - 1)
                y[:, t, d] = q[:, t, d] * (hd[: s + 1] * x[:, t - np.arange(s + 1), d]).sum(axis=1)
        return y

    def direct_bwd(q, k, v, h, dy, gs):
        B, L, D = q.shape
        G, lh = h.shape
        x, dz = k * v, dy * q
        z = direct(np.ones_like(q), k, v, h, gs)
        dq = dy * z
        dx = np.zeros_like(q)
        dh = np.zeros_like(h)
        for d in range(D):
            g = d // gs
            for t in range(L):
                for s in range(min(lh, L - t)):
                    dx[:, t, d] += h[g, s] * dz[:, t + s, d]
                for s in range(min(lh, t + 1)):
                    dh[g, s] += (dz[:, t, d] * x[:, t - s, d]).sum()
        return dq, dx * v, dx * k, dh

    cases = [(1, 1, 2, 1, 1), (2, 5, 4, 2, 9), (1, 17, 6, 3, 4), (3, 9, 4, 4, 1), (1, 33, 8, 8, 32)]
    for B, L, D, gs, lh in cases:
        q, k, v, dy = (rng.standard_normal((B, L, D)) for _ in range(4))
        h = rng.standard_normal((D // gs, lh))
        y = oracle.conv_fwd_ref(q, k, v, h, gs)
        assert np.allclose(y, direct(q, k, v, h, gs), rtol=1e-12, atol=1e-12), (B, L, D, gs, lh)
        got = oracle.conv_bwd_ref(q, k, v, h, dy, gs)
        for a, b in zip(got, direct_bwd(q, k, v, h, dy, gs)):
            assert np.allclose(a, b, rtol=1e-11, atol=1e-11), (B, L, D, gs, lh)
    print("sanitized oracle ok", flush=True)
''')


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None or _runtime("libubsan.so") is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "libhyena_ref_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-o", lib, SRC],
                   check=True)
    env = dict(os.environ, LD_PRELOAD=os.path.realpath(asan), OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", CHILD, lib, ROOT], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "sanitized oracle ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
