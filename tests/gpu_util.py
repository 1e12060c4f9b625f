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
import math
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


# ---- backward --------------------------------------------------------------
# dq, dk, dv use the forward's bar with the envelope of the backward oracle
# on magnitudes; dh (fp32 output) |e| <= (u_in + (R + 256) 2^-24) env with
# u_in = 2^-7 + 2^-14 (bf16 inputs: dz and x each rounded once) or 4 2^-24
# (fp32), R the partial rows summed, plus the gate.

def bwd_refs(q, k, v, h, dy, gs):
    """(oracle gradients, the same on magnitudes) for CPU or GPU tensors."""
    a = [to_np(t) for t in (q, k, v, h, dy)]
    ref = oracle.conv_bwd_ref(*a, gs)
    env = oracle.conv_bwd_ref(*[np.abs(x) for x in a], gs)
    return ref, env


def check_dh(got, ref, env, dtype, rows, what):
    got = to_np(got)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    gate = (1e-2 if dtype == torch.bfloat16 else 1e-5) * scale
    u_in = 2.0 ** -7 + 2.0 ** -14 if dtype == torch.bfloat16 else 4 * 2.0 ** -24
    bound = (u_in + (rows + 256) * 2.0 ** -24) * env + TINY
    assert float(np.max(err)) <= gate, "%s: dh max err %.3e > gate %.3e" % (what, np.max(err), gate)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, "%s: dh bound broken at %s" % (what, bad[0])


def check_bwd(grads, ref, env, l_h, dtype, rows, what):
    for name, g, r, e in zip(("dq", "dk", "dv"), grads[:3], ref[:3], env[:3]):
        check(to_np(g), r, e, l_h, dtype, "%s %s" % (what, name))
    check_dh(grads[3], ref[3], env[3], dtype, rows, what)


def bwd_rows(B, L, D, gs, l_h, dtype):
    """Partial rows the filter gradient sums (from the workspace size)."""
    n = hc.bwd_workspace_bytes(B, L, D, gs, l_h, hc.DTYPE_BF16 if dtype == torch.bfloat16 else hc.DTYPE_F32)
    return max(1, n // ((D // 16) * l_h * 4))


# ---- long filters (FFT convolution) ------------------------------------------
# The FFT path's rounding error is not local.  Per channel d of group g and
# transform length N (fp32 transforms for both I/O types):
#     |y - y_ref| <= r |y_ref| + |q| * 3 e sqrt(N) ||h_g||_2 ||x_d||_2,
#     e = (log2 N + 2) * 7 * 2^-24,
# r = 2^-8 (bf16 output rounding) or 2^-24 (fp32): the norm-wise error of a
# radix-2 FFT (about 7 units of rounding per level with accurate twiddles,
# log2 N levels plus the two twiddle passes of the split) through the forward
# transforms of x and h, the product and the inverse.  The spec gate is
# applied as well.

def transform_len(L, l_h):
    n = L + min(l_h, L) - 1
    return 1 << max(2, (n - 1).bit_length())


def register_fed_forms(L, D, gs, l_h):
    """The register-fed forms the long-filter plan takes: "rows" (the row and
    output kernels, rows3 and out3 under the three-level split), "mid" (the
    three-level middle passes), "col1" (single column) and "bwd1" (the
    backward's single column).  Each needs a transform of 32 to 256 points
    whose tile of pairs (at most 64, at most 4096 values with the backward's
    two sequences per pair, no wider than the pairs there are) holds exactly
    4096 values, 16 for each of 256 threads."""
    N = transform_len(L, l_h)
    log_n = N.bit_length() - 1
    three = log_n > 16
    if three:  # N1 N2 N3, every transform at most 256 points
        log1 = (log_n + 2) // 3
        log2 = (log_n - log1 + 1) // 2
        log3 = log_n - log1 - log2
    else:
        log1, log2, log3 = (log_n + 1) // 2, log_n // 2, 0

    def full(log_m, seqs, pairs):
        m = 1 << log_m
        P = 64
        while P > 1 and seqs * m * P > 4096:
            P //= 2
        while P > 1 and P // 2 >= pairs:
            P //= 2
        return 5 <= log_m <= 8 and seqs * m * P == 4096

    pairs = max(D // 2, (D // gs + 1) // 2)
    return {
        "rows": full(log3 if three else log2, 1, pairs),
        "mid": three and full(log2, 1, pairs),
        "col1": gs % 2 == 0 and full(log1, 1, pairs),
        "bwd1": gs % 2 == 0 and full(log1, 2, D // 2),
    }


def run_long(q, k, v, h, gs, pad=16):
    n = q.numel()
    big = torch.full((n + 2 * pad,), 7.0, dtype=q.dtype, device=q.device)
    out = big[pad:pad + n].view(q.shape)
    out.fill_(float("nan"))
    hc.conv_fwd_long(q, k, v, h, gs, out=out)
    torch.cuda.synchronize()
    assert torch.all(big[:pad] == 7.0) and torch.all(big[pad + n:] == 7.0), "write outside out"
    return out


def check_long(y, q, k, v, h, gs, dtype, what=""):
    """Gate and the norm-wise FFT bound against the fp64 oracle (CPU tensors)."""
    qn, kn, vn, hn = (to_np(t) for t in (q, k, v, h))
    ref = oracle.conv_fwd_ref(qn, kn, vn, hn, gs)
    y = to_np(y)
    assert np.all(np.isfinite(y)), what
    err = np.abs(y - ref)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    gate = (1e-2 if dtype == torch.bfloat16 else 1e-5) * scale
    assert float(np.max(err)) <= gate, "%s: max err %.3e > gate %.3e" % (what, np.max(err), gate)
    B, L, D = qn.shape
    N = transform_len(L, hn.shape[1])
    e = (math.log2(N) + 2) * 7 * 2.0 ** -24
    x = kn * vn
    xn = np.sqrt(np.sum(x * x, axis=1))                   # [B, D]
    hnorm = np.sqrt(np.sum(hn * hn, axis=1))[np.arange(D) // gs]  # [D]
    r = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -24
    bound = r * np.abs(ref) + np.abs(qn) * (3 * e * math.sqrt(N) * hnorm[None, None, :] * xn[:, None, :]) + TINY
    bad = np.argwhere(err > bound)
    assert bad.size == 0, "%s: FFT bound broken at %s" % (what, bad[0])
    return float(np.max(err)) / scale if scale else 0.0


# ---- long-filter backward (FFT) ---------------------------------------------
# Bars, per channel d of group g, batch row b and transform length N, with e
# and r as for the forward: dq: r |ref| + |dy| 3 e sqrt(N) ||h_g|| ||x_bd||;
# dk (dv): r |ref| + |v| (|k|) 3 e sqrt(N) ||h_g|| ||dz_bd||; dh: 3 e sqrt(N)
# sum_{b, d in g} ||dz_bd|| ||x_bd||; gates 1e-2 (bf16) / 1e-5 (fp32) of
# max|ref| for dq, dk, dv and 1e-5 for dh (fp32 output).

def run_long_bwd(q, k, v, h, dy, gs, pad=16, **need):
    """hyena_conv_bwd_long into NaN-filled outputs with canaries around each."""
    B, L, D = q.shape
    G, l_h = h.shape
    n = q.numel()
    bigs, outs = [], []
    for shape, dt, cnt in (((B, L, D), q.dtype, n), ((B, L, D), q.dtype, n), ((B, L, D), q.dtype, n),
                           ((G, l_h), torch.float32, G * l_h)):
        big = torch.full((cnt + 2 * pad,), 7.0, dtype=dt, device=DEV)
        out = big[pad:pad + cnt].view(shape)
        out.fill_(float("nan"))
        bigs.append(big)
        outs.append(out)
    want = [need.get("dq", True), need.get("dkv", True), need.get("dkv", True), need.get("dh", True)]
    code = hc.DTYPE_BF16 if q.dtype == torch.bfloat16 else hc.DTYPE_F32
    ws_n = hc.bwd_long_workspace_bytes(B, L, D, gs, l_h, code)
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=DEV)
    ws.fill_(0xff)  # contents need not be initialised
    ptr = lambda t, w: t.data_ptr() if w else None
    st = hc.lib().hyena_conv_bwd_long(q.data_ptr(), k.data_ptr(), v.data_ptr(), h.data_ptr(), dy.data_ptr(),
                                      B, L, D, gs, l_h, *[ptr(o, w) for o, w in zip(outs, want)], code,
                                      ws.data_ptr(), ws_n, torch.cuda.current_stream().cuda_stream)
    assert st == 0, hc.strerror(st)
    torch.cuda.synchronize()
    for big, cnt in zip(bigs, (n, n, n, G * l_h)):
        assert torch.all(big[:pad] == 7.0) and torch.all(big[pad + cnt:] == 7.0), "write outside an output"
    return [o if w else None for o, w in zip(outs, want)]


def check_long_bwd(got, q, k, v, h, dy, gs, dtype, what=""):
    """Gates and norm-wise FFT bounds of all four gradients against the fp64 oracle."""
    qn, kn, vn, hn, dyn = (to_np(t) for t in (q, k, v, h, dy))
    ref = oracle.conv_bwd_ref(qn, kn, vn, hn, dyn, gs)
    B, L, D = qn.shape
    N = transform_len(L, hn.shape[1])
    e = (math.log2(N) + 2) * 7 * 2.0 ** -24
    r = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -24
    x = kn * vn
    dz = dyn * qn
    xn = np.sqrt(np.sum(x * x, axis=1))                    # [B, D]
    zn = np.sqrt(np.sum(dz * dz, axis=1))                  # [B, D]
    hnorm = np.sqrt(np.sum(hn * hn, axis=1))[np.arange(D) // gs]  # [D]
    k3 = 3 * e * math.sqrt(N)
    rel = {}
    bounds = {
        "dq": np.abs(dyn) * (k3 * hnorm[None, None, :] * xn[:, None, :]),
        "dk": np.abs(vn) * (k3 * hnorm[None, None, :] * zn[:, None, :]),
        "dv": np.abs(kn) * (k3 * hnorm[None, None, :] * zn[:, None, :]),
    }
    for i, name in enumerate(("dq", "dk", "dv")):
        if got[i] is None:
            continue
        y = to_np(got[i])
        assert np.all(np.isfinite(y)), "%s %s" % (what, name)
        err = np.abs(y - ref[i])
        scale = float(np.max(np.abs(ref[i]))) if ref[i].size else 0.0
        gate = (1e-2 if dtype == torch.bfloat16 else 1e-5) * scale
        assert float(np.max(err, initial=0.0)) <= gate, "%s %s: max err %.3e > gate %.3e" % (
            what, name, np.max(err), gate)
        bad = np.argwhere(err > r * np.abs(ref[i]) + bounds[name] + TINY)
        assert bad.size == 0, "%s %s: FFT bound broken at %s" % (what, name, bad[0])
        rel[name] = float(np.max(err, initial=0.0)) / scale if scale else 0.0
    if got[3] is not None:
        dh = to_np(got[3])
        assert np.all(np.isfinite(dh)), "%s dh" % what
        err = np.abs(dh - ref[3])
        scale = float(np.max(np.abs(ref[3]))) if ref[3].size else 0.0
        assert float(np.max(err, initial=0.0)) <= 1e-5 * scale + TINY, "%s dh: max err %.3e > gate %.3e" % (
            what, np.max(err), 1e-5 * scale)
        G = D // gs
        terms = (zn * xn).sum(axis=0).reshape(G, gs).sum(axis=1)  # [G]
        bad = np.argwhere(err > k3 * terms[:, None] + TINY)
        assert bad.size == 0, "%s dh: FFT bound broken at %s" % (what, bad[0])
        taps = min(hn.shape[1], L)
        assert np.all(dh[:, taps:] == 0.0), "%s dh: taps past the sequence must be zero" % what
        rel["dh"] = float(np.max(err, initial=0.0)) / scale if scale else 0.0
    return rel
