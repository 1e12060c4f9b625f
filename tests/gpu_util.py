"""Shared helpers of the GPU parity tests: device setup and the accuracy bar.

The bar (applied element by element against the fp64 oracle):

bf16 I/O -- the gate every result must pass is
    max|y - y_ref| <= 1e-2 * max|y_ref|.
The library rounds k*v once to bf16 (relative error <= 2^-8), sums in fp32
(<= l_h * 2^-24 relative to the sum of magnitudes) and rounds the gated
output once to bf16 (<= 2^-8).  So each element must also satisfy
    |y - y_ref| <= 2^-8 |y_ref| + (2^-8 (1 + 2^-8) + l_h 2^-23) * env + tiny,
with env = |q| (|h| * |k v|), the same operator on magnitudes.
fp32 I/O -- gate max|y - y_ref| <= 1e-5 * max|y_ref|; elementwise
    |y - y_ref| <= 2^-24 |y_ref| + (l_h + 4) 2^-23 * env + tiny.
"""
import sys

import numpy as np
import torch

import gated_convolution_sequence_amd as hc
import oracle

DEV = torch.device("cuda:0")
TINY = 1e-30


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def nan_like(t: torch.Tensor) -> torch.Tensor:
    return torch.full_like(t, float("nan"))


def ref_and_envelope(q, k, v, h, gs):
    """(oracle output, |q| (|h| * |k v|)) as float64 numpy arrays."""
    qn, kn, vn, hn = to_np(q), to_np(k), to_np(v), to_np(h)
    ref = oracle.conv_fwd_ref(qn, kn, vn, hn, gs)
    env = oracle.conv_fwd_ref(np.abs(qn), np.abs(kn), np.abs(vn), np.abs(hn), gs)
    return ref, env


def check(y: np.ndarray, ref: np.ndarray, env: np.ndarray, l_h: int, dtype: torch.dtype,
          what: str = "") -> float:
    """Assert the gate and the elementwise bound; returns max|y - ref| / max|ref|."""
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), "%s: non-finite output" % what
    err = np.abs(y - ref)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if dtype == torch.bfloat16:
        gate = 1e-2 * scale
        elem = 2.0 ** -8 * np.abs(ref) + (2.0 ** -8 * (1 + 2.0 ** -8) + l_h * 2.0 ** -23) * env + TINY
    else:
        gate = 1e-5 * scale
        elem = 2.0 ** -24 * np.abs(ref) + (l_h + 4) * 2.0 ** -23 * env + TINY
    emax = float(np.max(err)) if err.size else 0.0
    assert emax <= gate, "%s: max err %.3e > gate %.3e" % (what, emax, gate)
    bad = err > elem
    if np.any(bad):
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: elementwise bound broken at %s: y=%r ref=%r env=%r" % (
            what, tuple(i), y[tuple(i)], ref[tuple(i)], env[tuple(i)]))
    return emax / scale if scale > 0 else 0.0


def run(q, k, v, h, gs, span=0, pad=16):
    """Forward through the C ABI into a NaN-filled output with canaries on both sides."""
    n = q.numel()
    big = torch.full((n + 2 * pad,), 7.0, dtype=q.dtype, device=q.device)
    out = big[pad:pad + n].view(q.shape)
    out.fill_(float("nan"))
    hc.conv_fwd(q, k, v, h, gs, out=out, span_chunks=span)
    torch.cuda.synchronize()
    assert torch.all(big[:pad] == 7.0) and torch.all(big[pad + n:] == 7.0), "write outside out"
    return out
