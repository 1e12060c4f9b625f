"""GPU parity of the halo-in forward (one shard of a longer sequence).

hyena_conv_fwd_halo runs rows [s, L) of a sequence given the rows before s
as k_prev / v_prev.  Its output must equal rows [s, L) of the forward over
the whole sequence: bitwise when s is a multiple of the 64-row chunk (the
same fp32 sums in the same order), and within the accuracy bar of the fp64
oracle for any s and any prefix length.
"""
import numpy as np
import pytest
import torch

import gated_convolution_sequence_amd as hc
from gpu_util import DEV, check, log, nan_like, ref_and_envelope, to_np
from workloads import gaussian_inputs

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    hc.lib()


def _run(q, k, v, h, gs, span=0, kp=None, vp=None):
    out = nan_like(q)
    hc.conv_fwd(q, k, v, h, gs, out=out, span_chunks=span, k_prev=kp, v_prev=vp)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("l_h,split,span", [
    (7, 256, 0), (128, 512, 0), (128, 640, 1), (65, 192, 2), (128, 64, 0), (33, 1024, 4),
    (100, 300, 0), (128, 1000, 2), (2, 65, 1)])
def test_shard_with_prefix_matches_the_whole_sequence(dt, l_h, split, span):
    log("halo %s l_h=%d split=%d span=%d" % (dt, l_h, split, span))
    dtype = DTYPES[dt]
    B, L, D, gs = 2, 1600, 256, 16
    q, k, v, h = (t.to(DEV) for t in gaussian_inputs(B, L, D, gs, l_h, dtype, seed=split + l_h))
    full = _run(q, k, v, h, gs, span)
    Pn = min(l_h - 1, split)  # rows before 0 are zero in both runs
    sl = lambda a: a[:, split:].contiguous()
    kp, vp = k[:, split - Pn:split].contiguous(), v[:, split - Pn:split].contiguous()
    shard = _run(sl(q), sl(k), sl(v), h, gs, span, kp, vp)
    if split % 64 == 0:
        assert torch.equal(shard, full[:, split:])
    ref, env = ref_and_envelope(q.cpu(), k.cpu(), v.cpu(), h.cpu(), gs)
    check(to_np(shard), ref[:, split:], env[:, split:], l_h, dtype, "halo shard")


@pytest.mark.parametrize("Pn", [0, 1, 10, 126, 127, 128, 300])
def test_prefix_length(Pn):
    """Short prefixes mean zeros before them; long ones are read only in their last l_h-1 rows."""
    log("halo prefix P=%d" % Pn)
    dtype, l_h, gs = torch.bfloat16, 128, 16
    B, L, D = 1, 700, 128
    qa, ka, va, h = gaussian_inputs(B, Pn + L, D, gs, l_h, dtype, seed=Pn)
    q, k, v = (a[:, Pn:].contiguous().to(DEV) for a in (qa, ka, va))
    kp = ka[:, :Pn].contiguous().to(DEV) if Pn else None
    vp = va[:, :Pn].contiguous().to(DEV) if Pn else None
    y = _run(q, k, v, h.to(DEV), gs, 0, kp, vp)
    ref, env = ref_and_envelope(qa, ka, va, h, gs)  # the concatenated sequence
    check(to_np(y), ref[:, Pn:], env[:, Pn:], l_h, dtype, "prefix %d" % Pn)
    if Pn == 0:
        assert torch.equal(y, _run(q, k, v, h.to(DEV), gs))


def test_two_shards_rebuild_the_mr_workload_row_by_row():
    """B=1, L=8192, D=4096, l_h=128 split in two at row 4096, as on two GPUs."""
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS["mr"]
    log("mr in two shards")
    q, k, v, h = make_inputs(w, DEV)
    full = _run(q, k, v, h, w.group_size)
    s = w.L // 2
    first = _run(q[:, :s].contiguous(), k[:, :s].contiguous(), v[:, :s].contiguous(), h, w.group_size)
    second = _run(q[:, s:].contiguous(), k[:, s:].contiguous(), v[:, s:].contiguous(), h, w.group_size,
                  0, k[:, s - (w.l_h - 1):s].contiguous(), v[:, s - (w.l_h - 1):s].contiguous())
    assert torch.equal(torch.cat([first, second], dim=1), full)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("gs,l_h,split,Pn", [(1, 7, 256, 6), (3, 8, 100, 7), (2, 4, 65, 2), (1, 1, 300, 0),
                                             (5, 6, 700, 40)])
def test_off_tile_short_filter_shard_with_prefix(dt, gs, l_h, split, Pn):
    """Group sizes off the 16-channel tile with at most 8 taps take the direct
    kernel, which reads the rows before row 0 from the prefix.  Its sums do
    not depend on where a span starts, so a shard with its prefix gives the
    whole sequence's bits once the prefix covers the filter (a shorter one
    means zeros before it, checked against the oracle)."""
    log("halo direct %s gs=%d l_h=%d split=%d P=%d" % (dt, gs, l_h, split, Pn))
    dtype = DTYPES[dt]
    B, L, D = 2, 1000, 120
    q, k, v, h = (t.to(DEV) for t in gaussian_inputs(B, L, D, gs, l_h, dtype, seed=split + l_h + gs))
    full = _run(q, k, v, h, gs)
    sl = lambda a: a[:, split:].contiguous()
    kp = k[:, split - Pn:split].contiguous() if Pn else None
    vp = v[:, split - Pn:split].contiguous() if Pn else None
    shard = _run(sl(q), sl(k), sl(v), h, gs, 0, kp, vp)
    if Pn >= l_h - 1:
        assert torch.equal(shard, full[:, split:])
    qc, kc, vc = (a[:, split - Pn:].cpu() for a in (q, k, v))
    ref, env = ref_and_envelope(qc, kc, vc, h.cpu(), gs)
    check(to_np(shard), ref[:, Pn:], env[:, Pn:], l_h, dtype, "halo direct shard")
