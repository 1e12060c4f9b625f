"""Seeded random shapes through every entry point, against the fp64 oracle.

The fixed edge lists of the other GPU suites pick the seams by hand (chunk,
block and slab boundaries, history depths, spans).  Here a fixed-seed draw
of shapes -- batch rows, ragged lengths, widths, group sizes, filter
lengths, requested spans, both dtypes -- goes through the same C ABI and is
held to the same bars (tests/gpu_util.py), so combinations the lists do not
name are covered too.  The draw is fixed: the cases are the same on every
run.
"""
import numpy as np
import pytest
import torch

import gated_convolution_sequence_amd as hc
from gpu_util import (DEV, bwd_refs, bwd_rows, check, check_bwd, check_long, check_long_bwd, log, ref_and_envelope,
                      register_fed_forms, run, run_long, run_long_bwd, to_np)
from workloads import gaussian_inputs, normal_activation

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}
N_CASES = 12


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    hc.lib()
    yield
    torch.cuda.synchronize()


def _draw(kind, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(N_CASES):
        dt = str(rng.choice(["bf16", "f32"]))
        B = int(rng.integers(1, 4))
        L = int(rng.choice([rng.integers(1, 130), rng.integers(130, 3000)]))
        if kind == "grouped":
            gs = int(rng.choice([16, 32, 48, 64]))
            D = gs * int(rng.integers(1, max(2, 384 // gs) + 1))
            l_h = int(rng.integers(1, 129))
            span = int(rng.choice([0, 1, 2, 4, 8, 16, 32]))
            cases.append((dt, B, L, D, gs, l_h, span))
        elif kind == "chunk_direction":
            gs = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 24]))
            unit = np.lcm(gs, 8 if dt == "bf16" else 4)  # whole 16-byte rows
            D = int(unit * rng.integers(1, max(2, 192 // unit) + 1))
            l_h = int(rng.integers(1, 129))
            span = int(rng.choice([0, 4, 8, 16]))
            cases.append((dt, B, L, D, gs, l_h, span))
        elif kind == "backward":
            gs = int(rng.choice([16, 32, 48]))
            D = gs * int(rng.integers(1, max(2, 192 // gs) + 1))
            L = min(L, 1500)
            l_h = int(rng.integers(1, 129))
            cases.append((dt, B, L, D, gs, l_h, 0))
        elif kind == "backward_off_tile":
            gs = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 24]))
            unit = np.lcm(gs, 8 if dt == "bf16" else 4)  # whole 16-byte rows
            D = int(unit * rng.integers(1, max(2, 192 // unit) + 1))
            L = min(L, 1500)
            l_h = int(rng.integers(1, 129))
            cases.append((dt, B, L, D, gs, l_h, 0))
        elif kind == "halo":
            gs = int(rng.choice([1, 3, 8, 16, 32]))
            unit = np.lcm(gs, 8 if dt == "bf16" else 4) if gs % 16 else gs
            D = int(unit * rng.integers(1, max(2, 192 // unit) + 1))
            L = max(L, 2)
            l_h = int(rng.integers(1, 129))
            # (the span column carries the prefix length P)
            cases.append((dt, B, L, D, gs, l_h, int(rng.integers(0, 200))))
        elif kind == "long_wide":
            # widths whose pair tiles fill 4096 values: the register-fed forms
            gs = int(rng.choice([2, 4, 8, 16]))
            B = int(rng.integers(1, 3))
            L = int(rng.integers(1000, 3001))
            D = int(2 * rng.integers(64, 129))
            D -= D % gs
            l_h = int(rng.integers(1, 3001))
            cases.append((dt, B, L, D, gs, l_h, 0))
        else:  # long filters (forward; "long_backward": shorter sequences)
            gs = int(rng.choice([1, 2, 3, 4, 8, 16]))
            D = int(np.lcm(gs, 2) * rng.integers(1, max(2, 48 // np.lcm(gs, 2)) + 1))
            l_h = int(rng.integers(1, 5000))
            if kind == "long_backward":
                L = min(L, 2000)
            cases.append((dt, B, L, D, gs, l_h, 0))
    return cases


def _ids(cases):
    return ["%s-B%d-L%d-D%d-gs%d-lh%d-s%d" % c for c in cases]


GROUPED = _draw("grouped", 101)
CHUNK_DIR = _draw("chunk_direction", 202)
BACKWARD = _draw("backward", 303)
LONG = _draw("long", 404)
BACKWARD_OFF = _draw("backward_off_tile", 505)
HALO = _draw("halo", 606)
LONG_BWD = _draw("long_backward", 707)
LONG_WIDE = _draw("long_wide", 808)


def test_wide_draw_reaches_the_register_fed_forms():
    """Most wide long-filter cases take the register-fed row and column forms."""
    forms = [register_fed_forms(L, D, gs, l_h) for _, _, L, D, gs, l_h, _ in LONG_WIDE]
    assert sum(f["rows"] for f in forms) >= N_CASES // 2
    assert sum(f["col1"] and f["bwd1"] for f in forms) >= N_CASES // 2


@pytest.mark.parametrize("dt,B,L,D,gs,l_h,span", GROUPED, ids=_ids(GROUPED))
def test_random_grouped_forward(dt, B, L, D, gs, l_h, span):
    log("random grouped %s B=%d L=%d D=%d gs=%d l_h=%d span=%d" % (dt, B, L, D, gs, l_h, span))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=B * 100003 + L * 7 + D + l_h)
    y = run(q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV), gs, span)
    ref, env = ref_and_envelope(q, k, v, h, gs)
    check(to_np(y), ref, env, l_h, dtype, "random grouped")


@pytest.mark.parametrize("dt,B,L,D,gs,l_h,span", CHUNK_DIR, ids=_ids(CHUNK_DIR))
def test_random_chunk_direction_forward(dt, B, L, D, gs, l_h, span):
    log("random chunk-direction %s B=%d L=%d D=%d gs=%d l_h=%d span=%d" % (dt, B, L, D, gs, l_h, span))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=B * 100019 + L * 11 + D + l_h)
    y = run(q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV), gs, span)
    ref, env = ref_and_envelope(q, k, v, h, gs)
    check(to_np(y), ref, env, l_h, dtype, "random chunk-direction")


@pytest.mark.parametrize("dt,B,L,D,gs,l_h,span", BACKWARD, ids=_ids(BACKWARD))
def test_random_backward(dt, B, L, D, gs, l_h, span):
    log("random backward %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=B * 100043 + L * 13 + D + l_h)
    dy = normal_activation((B, L, D), dtype, "cpu", seed=L + D + 3)
    grads = hc.conv_bwd(*[t.to(DEV) for t in (q, k, v, h, dy)], gs)
    torch.cuda.synchronize()
    ref, env = bwd_refs(q, k, v, h, dy, gs)
    check_bwd(grads, ref, env, l_h, dtype, bwd_rows(B, L, D, gs, l_h, dtype), "random backward")


@pytest.mark.parametrize("dt,B,L,D,gs,l_h,span", LONG, ids=_ids(LONG))
def test_random_long_filter(dt, B, L, D, gs, l_h, span):
    log("random long filter %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=B * 100057 + L * 17 + D + l_h)
    y = run_long(q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV), gs)
    check_long(y, q, k, v, h, gs, dtype, "random long filter")


@pytest.mark.parametrize("dt,B,L,D,gs,l_h,span", BACKWARD_OFF, ids=_ids(BACKWARD_OFF))
def test_random_backward_off_tile(dt, B, L, D, gs, l_h, span):
    """Group sizes off the 16-channel tile: the direct kernels (8 taps or
    fewer) or the chunk-direction kernel and the lag products (longer)."""
    log("random backward off tile %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=B * 100069 + L * 19 + D + l_h)
    dy = normal_activation((B, L, D), dtype, "cpu", seed=L + D + 5)
    grads = hc.conv_bwd(*[t.to(DEV) for t in (q, k, v, h, dy)], gs)
    torch.cuda.synchronize()
    ref, env = bwd_refs(q, k, v, h, dy, gs)
    code = hc.DTYPE_BF16 if dtype == torch.bfloat16 else hc.DTYPE_F32
    rows = max(1, hc.bwd_workspace_bytes(B, L, D, gs, l_h, code) // (D * l_h * 4)) * gs
    check_bwd(grads, ref, env, l_h, dtype, rows, "random backward off tile")


@pytest.mark.parametrize("dt,B,L,D,gs,l_h,P", HALO, ids=_ids(HALO))
def test_random_history_prefix(dt, B, L, D, gs, l_h, P):
    """A shard of a longer sequence: the last L rows of P + L, with the first
    P rows passed as the prefix, against the oracle on the whole sequence."""
    log("random prefix %s B=%d L=%d D=%d gs=%d l_h=%d P=%d" % (dt, B, L, D, gs, l_h, P))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, P + L, D, gs, l_h, dtype, seed=B * 100103 + L * 23 + D + l_h + P)
    qd, kd, vd, hd = (t.to(DEV) for t in (q, k, v, h))
    sl = lambda a: a[:, P:].contiguous()
    out = torch.full_like(sl(qd), float("nan"))
    if P:
        hc.conv_fwd(sl(qd), sl(kd), sl(vd), hd, gs, out=out, k_prev=kd[:, :P].contiguous(),
                    v_prev=vd[:, :P].contiguous())
    else:
        hc.conv_fwd(sl(qd), sl(kd), sl(vd), hd, gs, out=out)
    torch.cuda.synchronize()
    ref, env = ref_and_envelope(q, k, v, h, gs)
    check(to_np(out), ref[:, P:], env[:, P:], l_h, dtype, "random prefix")


@pytest.mark.parametrize("dt,B,L,D,gs,l_h,span", LONG_BWD, ids=_ids(LONG_BWD))
def test_random_long_filter_backward(dt, B, L, D, gs, l_h, span):
    """hyena_conv_bwd_long: all four gradients against the fp64 backward oracle."""
    log("random long backward %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=B * 7919 + L * 31 + D + 3 * l_h)
    dy = normal_activation((B, L, D), dtype, "cpu", seed=L + 2 * l_h + 1)
    got = run_long_bwd(*(t.to(DEV) for t in (q, k, v, h, dy)), gs)
    check_long_bwd(got, q, k, v, h, dy, gs, dtype, "random long backward")


@pytest.mark.parametrize("dt,B,L,D,gs,l_h,span", LONG_WIDE, ids=_ids(LONG_WIDE))
def test_random_long_filter_wide(dt, B, L, D, gs, l_h, span):
    """Widths that fill the FFT tiles (register-fed forms), forward and backward."""
    log("random wide long filter %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=B * 6007 + L * 37 + D + 5 * l_h)
    dy = normal_activation((B, L, D), dtype, "cpu", seed=L + 3 * l_h + 2)
    qd, kd, vd, hd = (t.to(DEV) for t in (q, k, v, h))
    y = run_long(qd, kd, vd, hd, gs)
    check_long(y, q, k, v, h, gs, dtype, "random wide long filter")
    got = run_long_bwd(qd, kd, vd, hd, dy.to(DEV), gs)
    check_long_bwd(got, q, k, v, h, dy, gs, dtype, "random wide long backward")
