"""hyena_conv_bwd_noalloc: the backward without a caller workspace and
without device allocation (its partial filter gradients go to a fixed device
array of the library).

On the GPU it must give the same bits as hyena_conv_bwd with a workspace on
the same inputs, on two calls in a row (the second with a smaller input, so
that it runs on the scratch contents the first call left), in bf16 and
fp32, on and off the 16-channel grouping.  On the CPU, a problem that needs
more than the fixed array is refused before any HIP call.
"""
import ctypes

import pytest
import torch

import gated_convolution_sequence_amd as hc
from workloads import gaussian_inputs

SCRATCH = 16 << 20


def test_scratch_size_is_stated():
    assert hc.lib().hyena_conv_scratch_bytes() == SCRATCH


def test_too_large_a_problem_is_refused_on_the_host():
    # B=8, L=32768, D=4096, 16-channel groups, l_h=128: 32 MiB of partial rows
    need = hc.bwd_workspace_bytes(8, 32768, 4096, 16, 128)
    assert need > SCRATCH
    a = 1 << 40  # fake device addresses: the call must return before touching them
    n = 8 * 32768 * 4096 * 2
    ptrs = [a + i * (n + (1 << 20)) for i in range(9)]
    st = hc.lib().hyena_conv_bwd_noalloc(*ptrs[:5], 8, 32768, 4096, 16, 128, *ptrs[5:8], ptrs[8],
                                         hc.DTYPE_BF16, None)
    assert st == -11 and "scratch" in hc.strerror(st)
    # the same sizes fit the fixed array once B is halved
    assert hc.bwd_workspace_bytes(4, 32768, 4096, 16, 128) == SCRATCH
    # without dh no scratch is needed; the other checks still come first
    assert hc.lib().hyena_conv_bwd_noalloc(None, *ptrs[1:5], 8, 32768, 4096, 16, 128, *ptrs[5:8], None,
                                           hc.DTYPE_BF16, None) == -1


def _grads(q, k, v, h, dy, gs, noalloc, need_dh=True):
    B, L, D = q.shape
    l_h = h.shape[1]
    code = hc.DTYPE_BF16 if q.dtype == torch.bfloat16 else hc.DTYPE_F32
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    dh = torch.full((D // gs, l_h), float("nan"), dtype=torch.float32, device=q.device) if need_dh else None
    s = torch.cuda.current_stream()
    ptr = lambda t: t.data_ptr() if t is not None else None
    if noalloc:
        st = hc.lib().hyena_conv_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), h.data_ptr(),
                                             dy.data_ptr(), B, L, D, gs, l_h, dq.data_ptr(), dk.data_ptr(),
                                             dv.data_ptr(), ptr(dh), code, s.cuda_stream)
    else:
        n = hc.bwd_workspace_bytes(B, L, D, gs, l_h, code)
        ws = torch.full((max(n, 16) // 4,), float("nan"), dtype=torch.float32, device=q.device)
        st = hc.lib().hyena_conv_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), h.data_ptr(), dy.data_ptr(),
                                     B, L, D, gs, l_h, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ptr(dh),
                                     ws.data_ptr(), n, code, s.cuda_stream)
    assert st == 0, hc.strerror(st)
    torch.cuda.synchronize()
    return dq, dk, dv, dh


CASES = [
    # (B, L, D, group_size, l_h, dtype): larger first, then smaller
    [(2, 16384, 4096, 16, 128, torch.bfloat16), (1, 1000, 64, 16, 65, torch.bfloat16)],
    [(1, 4096, 512, 32, 33, torch.float32), (2, 333, 48, 16, 7, torch.float32)],
    [(1, 8192, 4096, 1, 7, torch.bfloat16), (3, 500, 24, 3, 5, torch.bfloat16)],
]


@pytest.mark.gpu
@pytest.mark.parametrize("pair", CASES, ids=["grouped-bf16", "grouped-f32", "off-tile-bf16"])
def test_noalloc_backward_matches_the_workspace_entry(pair):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    dev = torch.device("cuda:0")
    for i, (B, L, D, gs, l_h, dtype) in enumerate(pair):
        print("noalloc call %d: B=%d L=%d D=%d gs=%d l_h=%d %s" % (i, B, L, D, gs, l_h, dtype), flush=True)
        q, k, v, h = (t.to(dev) for t in gaussian_inputs(B, L, D, gs, l_h, dtype, seed=B + L + D + l_h))
        dy = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(L), device=dev).to(dtype)
        ref = _grads(q, k, v, h, dy, gs, noalloc=False)
        got = _grads(q, k, v, h, dy, gs, noalloc=True)
        for name, a, b in zip(("dq", "dk", "dv", "dh"), got, ref):
            assert torch.isfinite(a).all(), (i, name)
            assert torch.equal(a, b), (i, name)
        # a call without dh needs no scratch and gives the bits of the same
        # call through the workspace entry
        ref = _grads(q, k, v, h, dy, gs, noalloc=False, need_dh=False)
        got = _grads(q, k, v, h, dy, gs, noalloc=True, need_dh=False)
        for name, a, b in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
            assert torch.equal(a, b), (i, name, "without dh")
