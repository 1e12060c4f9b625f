"""fp64 CPU oracle for y = q (.) (h * (k (.) v)).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
the two share no code: no kernels, headers, helpers or constant tables.

The arithmetic lives in ``hyena_ref.c`` (plain C, fp64, OpenMP over output
rows): the causal FIR definition from the page "04. hardware-aware convolution
kernels" (StripedHyena 2 explainer), section 1, first equation, gated as in
that page's Algorithm 1 (section 4), with one filter per channel group
(section 4, first bullet list); and its backward, the chain rule of that
definition term by term (the filter gradient being the global sum over
positions that the same page's section 7 describes).  See the C file for the
exact statements.

Every pin that ties this oracle to something other than itself lives in
``tests/test_oracle.py``; nothing here is left "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hyena_ref.c")
_LIB = os.path.join(_HERE, "libhyena_ref.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc into ``oracle/libhyena_ref.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
               "-Wall", "-Wextra", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.hyena_ref_fwd_f64.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, i64, dp]
        lib.hyena_ref_fwd_f64.restype = ctypes.c_int
        lib.hyena_ref_bwd_f64.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, dp, dp, dp, dp]
        lib.hyena_ref_bwd_f64.restype = ctypes.c_int
        lib.hyena_ref_num_threads.argtypes = []
        lib.hyena_ref_num_threads.restype = ctypes.c_int
        lib.hyena_ref_set_num_threads.argtypes = [ctypes.c_int]
        lib.hyena_ref_set_num_threads.restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads one oracle call uses."""
    return int(_load().hyena_ref_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads later oracle calls use (for timing; results do not depend on it)."""
    _load().hyena_ref_set_num_threads(int(n))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def conv_fwd_ref(q, k, v, h, group_size: int) -> np.ndarray:
    """y[b,t,d] = q[b,t,d] * sum_{s=0}^{min(t, l_h-1)} h[d//group_size, s] * k[b,t-s,d] * v[b,t-s,d].

    ``q``, ``k``, ``v``: [B, L, D]; ``h``: [D // group_size, l_h].  Inputs are
    widened to float64 (exact for bf16 and fp32 values); the result is float64.
    """
    q, k, v, h = _f64(q), _f64(k), _f64(v), _f64(h)
    if q.ndim != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, L, D] shape")
    B, L, D = q.shape
    if h.ndim != 2:
        raise ValueError("h must be [D // group_size, l_h]")
    G, l_h = h.shape
    if group_size < 1 or D % group_size != 0 or G != D // group_size:
        raise ValueError("h has %d filters; D=%d, group_size=%d" % (G, D, group_size))
    y = np.empty_like(q)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = _load().hyena_ref_fwd_f64(
        q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp),
        h.ctypes.data_as(dp), B, L, D, group_size, l_h, y.ctypes.data_as(dp))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return y


def conv_bwd_ref(q, k, v, h, dy, group_size: int):
    """(dq, dk, dv, dh) of y = q (.) (h * (k (.) v)) for upstream gradient dy, fp64.

    dq, dk, dv: [B, L, D]; dh: [D // group_size, l_h].
    """
    q, k, v, h, dy = _f64(q), _f64(k), _f64(v), _f64(h), _f64(dy)
    if q.ndim != 3 or any(a.shape != q.shape for a in (k, v, dy)):
        raise ValueError("q, k, v, dy must share one [B, L, D] shape")
    B, L, D = q.shape
    if h.ndim != 2:
        raise ValueError("h must be [D // group_size, l_h]")
    G, l_h = h.shape
    if group_size < 1 or D % group_size != 0 or G != D // group_size:
        raise ValueError("h has %d filters; D=%d, group_size=%d" % (G, D, group_size))
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    dh = np.empty_like(h)
    dp = ctypes.POINTER(ctypes.c_double)
    P = lambda a: a.ctypes.data_as(dp)
    rc = _load().hyena_ref_bwd_f64(P(q), P(k), P(v), P(h), P(dy), B, L, D, group_size, l_h,
                                   P(dq), P(dk), P(dv), P(dh))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return dq, dk, dv, dh
