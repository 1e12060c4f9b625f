"""GPU parity through the two entry points with the operator's own signature,
hyena_conv_fwd(q, k, v, h, B, L, D, group_size, l_h, out, stream) (bf16) and
hyena_conv_fwd_f32 (same arguments, fp32), called directly through ctypes,
not through the Python binding.

Each result is held to the bar of tests/gpu_util.py against the fp64 oracle
and must equal, bit for bit, the explicit-dtype entry point's result on the
same inputs (both take the library's default work split).
"""
import numpy as np
import pytest
import torch

import gated_convolution_sequence_amd as hc
from gpu_util import DEV, check, log, ref_and_envelope, to_np
from workloads import WORKLOADS, gaussian_inputs, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    hc.lib()
    yield
    torch.cuda.synchronize()


def _named(name, q, k, v, h, gs, stream=None, pad=16):
    """Call the named entry point into a NaN-filled output with canaries."""
    B, L, D = q.shape
    n = q.numel()
    big = torch.full((n + 2 * pad,), 7.0, dtype=q.dtype, device=q.device)
    out = big[pad:pad + n].view(q.shape)
    out.fill_(float("nan"))
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = getattr(hc.lib(), name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), h.data_ptr(), B, L, D, gs,
                                 h.shape[1], out.data_ptr(), s.cuda_stream)
    assert st == 0, hc.strerror(st)
    s.synchronize()
    assert torch.all(big[:pad] == 7.0) and torch.all(big[pad + n:] == 7.0), "write outside out"
    return out


def test_fwd_f32_tiny_se_full():
    w = WORKLOADS["tiny_se"]
    log("hyena_conv_fwd_f32: tiny_se")
    q, k, v, h = make_inputs(w, "cpu")
    qd, kd, vd, hd = (t.to(DEV) for t in (q, k, v, h))
    y = _named("hyena_conv_fwd_f32", qd, kd, vd, hd, w.group_size)
    ref, env = ref_and_envelope(q, k, v, h, w.group_size)
    rel = check(to_np(y), ref, env, w.l_h, torch.float32, "hyena_conv_fwd_f32 tiny_se")
    log("  rel err %.3e" % rel)
    assert torch.equal(y, hc.conv_fwd(qd, kd, vd, hd, w.group_size))


@pytest.mark.parametrize("name", ["se", "mr"])
def test_fwd_bf16_full_workload(name):
    w = WORKLOADS[name]
    log("hyena_conv_fwd: %s" % name)
    q, k, v, h = make_inputs(w, DEV)
    s = torch.cuda.Stream()  # a non-default stream, passed as the last argument
    torch.cuda.synchronize()
    y = _named("hyena_conv_fwd", q, k, v, h, w.group_size, stream=s)
    ref, env = ref_and_envelope(q, k, v, h, w.group_size)
    rel = check(to_np(y), ref, env, w.l_h, torch.bfloat16, "hyena_conv_fwd %s" % name)
    log("  rel err %.3e" % rel)
    assert torch.equal(y, hc.conv_fwd(q, k, v, h, w.group_size))


@pytest.mark.parametrize("name,dtype", [("hyena_conv_fwd", torch.bfloat16),
                                        ("hyena_conv_fwd_f32", torch.float32)])
@pytest.mark.parametrize("B,L,D,gs,l_h", [(2, 333, 48, 16, 65), (1, 1000, 72, 24, 9), (3, 70, 32, 1, 5),
                                          (1, 1, 16, 16, 128)])
def test_named_entry_points_small_shapes(name, dtype, B, L, D, gs, l_h):
    """Ragged lengths, a partial slab and group sizes off the 16-channel tile
    (the chunk-direction and direct kernels) through the named entry points."""
    log("%s B=%d L=%d D=%d gs=%d l_h=%d" % (name, B, L, D, gs, l_h))
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=L + D + l_h)
    y = _named(name, *(t.to(DEV) for t in (q, k, v, h)), gs)
    ref, env = ref_and_envelope(q, k, v, h, gs)
    check(to_np(y), ref, env, l_h, dtype, name)
    assert np.all(np.isfinite(to_np(y)))
