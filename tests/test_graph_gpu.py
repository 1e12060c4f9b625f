"""The entry points inside a captured HIP graph (torch.cuda.graph).

Serving loops and training steps replay captured graphs instead of issuing
launches one by one.  The library enqueues only kernels on the caller's
stream (no allocation, no memset at these sizes), so each entry point can be
captured.  Each graph is replayed several times; between replays the
program writes new inputs into the captured tensors eagerly and
synchronises, and every replay must equal an eager call on the same inputs
bit for bit.
"""
import pytest
import torch

import gated_convolution_sequence_amd as hc
from gpu_util import DEV, log
from workloads import gaussian_inputs, normal_activation

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    hc.lib()
    yield
    torch.cuda.synchronize()


def _replays(make_inputs, fn, n=3):
    """Capture fn(*static) once, then for n rounds: write new inputs eagerly,
    replay, compare with fn on fresh tensors."""
    static = [t.to(DEV) for t in make_inputs(0)]
    fn(*static)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn(*static)
    torch.cuda.synchronize()
    for r in range(1, n + 1):
        fresh = [t.to(DEV) for t in make_inputs(r)]
        for s, f in zip(static, fresh):
            s.copy_(f)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = fn(*fresh)
        torch.cuda.synchronize()
        got = outs if isinstance(outs, (tuple, list)) else (outs,)
        exp = want if isinstance(want, (tuple, list)) else (want,)
        for a, b in zip(got, exp):
            if a is None:
                continue
            assert torch.equal(a, b), "replay %d differs from the eager call" % r


@pytest.mark.parametrize("gs,l_h", [(16, 7), (16, 128), (1, 65), (3, 33)])
def test_forward_in_a_graph(gs, l_h):
    log("graph forward gs=%d l_h=%d" % (gs, l_h))
    B, L, D = 2, 1000, 96
    mk = lambda r: gaussian_inputs(B, L, D, gs, l_h, torch.bfloat16, seed=100 + r)
    _replays(mk, lambda q, k, v, h: hc.conv_fwd(q, k, v, h, gs))


def test_long_filter_in_a_graph():
    log("graph long filter")
    B, L, D, gs, l_h = 1, 2000, 64, 16, 2000
    ws = torch.empty(hc.long_workspace_bytes(B, L, D, gs, l_h), dtype=torch.uint8, device=DEV)
    mk = lambda r: gaussian_inputs(B, L, D, gs, l_h, torch.bfloat16, seed=200 + r)
    _replays(mk, lambda q, k, v, h: hc.conv_fwd_long(q, k, v, h, gs, workspace=ws))


def test_backward_in_a_graph():
    log("graph backward")
    B, L, D, gs, l_h = 1, 1000, 64, 16, 128

    def mk(r):
        q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, torch.bfloat16, seed=300 + r)
        return q, k, v, h, normal_activation((B, L, D), torch.bfloat16, "cpu", seed=400 + r)
    _replays(mk, lambda q, k, v, h, dy: hc.conv_bwd(q, k, v, h, dy, gs))


@pytest.mark.parametrize("gs", [16, 3])
def test_long_filter_backward_in_a_graph(gs):
    """hyena_conv_bwd_long (its dh tail is zeroed by a kernel: l_h > L here)."""
    log("graph long backward gs=%d" % gs)
    B, L, D, l_h = 2, 700, 48, 900
    ws = torch.empty(hc.bwd_long_workspace_bytes(B, L, D, gs, l_h), dtype=torch.uint8, device=DEV)

    def mk(r):
        q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, torch.bfloat16, seed=500 + r)
        return q, k, v, h, normal_activation((B, L, D), torch.bfloat16, "cpu", seed=600 + r)
    _replays(mk, lambda q, k, v, h, dy: hc.conv_bwd_long(q, k, v, h, dy, gs, workspace=ws))
