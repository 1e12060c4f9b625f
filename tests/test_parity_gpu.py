"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test here runs hyena_conv_fwd_ex on cuda:0 via the Python binding and
compares with oracle.conv_fwd_ref on the very same inputs, using the bar in
tests/gpu_util.py (spec gate plus an elementwise rounding bound), or
bitwise where every intermediate is exactly representable.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gated_convolution_sequence_amd as hc
import oracle
from gpu_util import DEV, check, log, nan_like, ref_and_envelope, run, to_np
from workloads import WORKLOADS, gaussian_inputs, integer_inputs, make_inputs

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    hc.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# shapes: ragged L, partial slabs, every history depth, spans that do not
# divide the chunk count, several groups per slab and groups wider than 16
# ---------------------------------------------------------------------------
EDGE = [
    # B, L, D, group_size, l_h, span
    (1, 1, 16, 16, 1, 0),
    (1, 6, 16, 16, 4, 0),
    (1, 63, 16, 16, 7, 0),
    (1, 64, 64, 16, 65, 0),
    (1, 65, 48, 16, 7, 0),
    (2, 127, 80, 16, 33, 1),
    (1, 129, 16, 16, 34, 1),
    (1, 1000, 64, 32, 128, 3),
    (3, 333, 96, 48, 65, 2),
    (1, 640, 128, 64, 66, 4),
    (1, 257, 16, 16, 97, 1),
    (1, 300, 32, 16, 98, 2),
    (2, 100, 32, 16, 2, 0),
    (1, 4096, 256, 16, 128, 7),
    (1, 2048, 1024, 16, 127, 0),
    (1, 515, 208, 16, 32, 5),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h,span", EDGE)
def test_edge_shapes_gaussian(dt, B, L, D, gs, l_h, span):
    log("edge %s B=%d L=%d D=%d gs=%d l_h=%d span=%d" % (dt, B, L, D, gs, l_h, span))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=B * 1000 + L + l_h)
    y = run(q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV), gs, span)
    ref, env = ref_and_envelope(q, k, v, h, gs)
    check(to_np(y), ref, env, l_h, dtype, "edge")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h,span", [
    (1, 6, 16, 16, 4, 0), (1, 1000, 64, 16, 128, 0), (2, 777, 96, 32, 7, 3),
    (1, 2049, 128, 16, 66, 1), (1, 4096, 4096, 16, 128, 0), (3, 130, 16, 16, 33, 1),
])
def test_integer_inputs_are_bitwise_exact(dt, B, L, D, gs, l_h, span):
    """q, k, v in {-1,0,1}, taps in {-2..2}: every partial sum is a small integer."""
    log("integer %s B=%d L=%d D=%d gs=%d l_h=%d span=%d" % (dt, B, L, D, gs, l_h, span))
    dtype = DTYPES[dt]
    q, k, v, h = integer_inputs(B, L, D, gs, l_h, dtype, seed=L + D)
    y = run(q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV), gs, span)
    ref = oracle.conv_fwd_ref(to_np(q), to_np(k), to_np(v), to_np(h), gs)
    assert np.array_equal(to_np(y), ref)


def test_worked_example_shape_matches_two_stage_blocks():
    """l = 6, l_h = 4 (the worked example's sizes) on 16 channels of one group."""
    log("worked example on GPU")
    L, l_h = 6, 4
    h = torch.tensor([[1.0, 2.0, 4.0, 8.0]], dtype=torch.bfloat16)
    v = torch.zeros(1, L, 16, dtype=torch.bfloat16)
    for d in range(16):
        v[0, d % L, d] = 1.0 + (d // L)  # channel d: impulse at time d % 6
    ones = torch.ones_like(v)
    y = to_np(run(ones.to(DEV), ones.to(DEV), v.to(DEV), h.to(DEV), 16))
    for d in range(16):
        t0, a = d % L, 1.0 + (d // L)
        expect = np.zeros(L)
        n = min(l_h, L - t0)
        expect[t0:t0 + n] = a * np.array([1.0, 2.0, 4.0, 8.0])[:n]
        assert np.array_equal(y[0, :, d], expect), d


@pytest.mark.parametrize("l_h", [1, 7, 64, 65, 66, 127, 128])
def test_impulses_on_chunk_seams_reproduce_the_filter(l_h):
    L, D = 600, 64
    seams = [0, 1, 63, 64, 65, 127, 128, 191, 192, 255, 256, 383, 384, 511, 512, L - 1]
    rng = np.random.default_rng(l_h)
    h = torch.tensor(rng.standard_normal((D // 16, l_h)), dtype=torch.bfloat16)
    v = torch.zeros(1, L, D, dtype=torch.bfloat16)
    for d in range(D):
        v[0, seams[d % len(seams)], d] = 1.0
    ones = torch.ones_like(v)
    for span in (0, 1, 3):
        log("impulses l_h=%d span=%d" % (l_h, span))
        y = to_np(run(ones.to(DEV), ones.to(DEV), v.to(DEV), h.to(DEV), 16, span))
        ref = oracle.conv_fwd_ref(to_np(ones), to_np(ones), to_np(v), to_np(h), 16)
        assert np.array_equal(y, ref)


def test_mr_last_tap_and_flat_filters():
    """A kernel missing the chunk n-2 block fails both by O(1)."""
    B, L, D, l_h = 1, 1024, 128, 128
    q, k, v, _ = gaussian_inputs(B, L, D, 16, l_h, torch.bfloat16, seed=5)
    last = torch.zeros(D // 16, l_h, dtype=torch.bfloat16)
    last[:, l_h - 1] = 1.0
    flat = torch.ones(D // 16, l_h, dtype=torch.bfloat16)
    ones = torch.ones_like(q)
    log("mr last tap")
    y = to_np(run(ones.to(DEV), ones.to(DEV), v.to(DEV), last.to(DEV), 16))
    ref = oracle.conv_fwd_ref(to_np(ones), to_np(ones), to_np(v), to_np(last), 16)
    assert np.array_equal(y, ref)  # a single exact term per output
    log("mr flat")
    y = to_np(run(q.to(DEV), k.to(DEV), v.to(DEV), flat.to(DEV), 16))
    ref, env = ref_and_envelope(q, k, v, flat, 16)
    check(y, ref, env, l_h, torch.bfloat16, "flat")


def test_deterministic_and_span_independent_rounding():
    """Bitwise identical across reruns; any span gives the same bits (same sum order)."""
    q, k, v, h = gaussian_inputs(2, 3000, 256, 16, 128, torch.bfloat16, seed=11)
    q, k, v, h = q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV)
    log("determinism")
    y0 = run(q, k, v, h, 16).clone()
    for span in (0, 0, 1, 2, 5, 47):
        y1 = run(q, k, v, h, 16, span)
        assert torch.equal(y0, y1), span


def test_batch_rows_and_causality():
    B, L, D, l_h = 3, 700, 64, 100
    q, k, v, h = gaussian_inputs(B, L, D, 16, l_h, torch.bfloat16, seed=12)
    k[1] = 0
    q, k, v, h = q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV)
    log("batch isolation and causality")
    y0 = run(q, k, v, h, 16).clone()
    assert torch.all(y0[1] == 0)
    t0 = 301
    v2 = v.clone()
    v2[:, t0] += 3.0
    y1 = run(q, k, v2, h, 16)
    assert torch.equal(y0[:, :t0], y1[:, :t0])
    assert torch.equal(y0[:, t0 + l_h:], y1[:, t0 + l_h:])


def test_stream_argument_is_honoured():
    q, k, v, h = gaussian_inputs(1, 512, 64, 16, 7, torch.bfloat16, seed=13)
    q, k, v, h = q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV)
    s = torch.cuda.Stream()
    out = nan_like(q)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        hc.conv_fwd(q, k, v, h, 16, out=out)
    s.synchronize()
    ref, env = ref_and_envelope(q.cpu(), k.cpu(), v.cpu(), h.cpu(), 16)
    check(to_np(out), ref, env, 7, torch.bfloat16, "stream")


# ---------------------------------------------------------------------------
# The workloads at full size
# ---------------------------------------------------------------------------

def test_tiny_se_fp32_full():
    w = WORKLOADS["tiny_se"]
    log("tiny_se full")
    q, k, v, h = make_inputs(w, "cpu")
    y = run(q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV), w.group_size)
    ref, env = ref_and_envelope(q, k, v, h, w.group_size)
    rel = check(to_np(y), ref, env, w.l_h, w.torch_dtype, "tiny_se")
    log("tiny_se rel err %.3e" % rel)


@pytest.mark.parametrize("name", ["se", "mr"])
def test_full_workload_every_element(name):
    w = WORKLOADS[name]
    log("%s full: generate" % name)
    q, k, v, h = make_inputs(w, DEV)
    y = run(q, k, v, h, w.group_size)
    log("%s full: oracle" % name)
    ref, env = ref_and_envelope(q, k, v, h, w.group_size)
    rel = check(to_np(y), ref, env, w.l_h, w.torch_dtype, name)
    log("%s rel err %.3e" % (name, rel))


def _window_check(q, k, v, h, y, w, b, t0, t1, c0, c1):
    """Exact sub-problem: rows [t0, t1) of channels [c0, c1) need l_h-1 rows of history."""
    gs = w.group_size
    s = max(0, t0 - (w.l_h - 1))
    sl = lambda a: a[b:b + 1, s:t1, c0:c1]
    hh = h[c0 // gs:c1 // gs]
    ref, env = ref_and_envelope(sl(q), sl(k), sl(v), hh, gs)
    got = to_np(sl(y))
    off = t0 - s
    check(got[:, off:], ref[:, off:], env[:, off:], w.l_h, w.torch_dtype,
          "%s b=%d t=[%d,%d) c=[%d,%d)" % (w.name, b, t0, t1, c0, c1))


def _sampled_checks(w, q, k, v, h, y, n_groups, seed):
    L, D = w.L, w.D
    mid = (1 << 31) // D  # the row where the element index reaches 2^31
    windows = [(0, 256), (L // 2 - 100, L // 2 + 37), (L - 256, L)]
    if mid + 128 <= L:
        windows.append((mid - 128, mid + 128))
    for b in sorted({0, w.B - 1}):
        for t0, t1 in windows:
            log("  window b=%d [%d,%d)" % (b, t0, t1))
            _window_check(q, k, v, h, y, w, b, t0, t1, 0, D)
    rng = np.random.default_rng(seed)
    groups = sorted({0, w.G - 1, *rng.choice(w.G, size=n_groups, replace=False).tolist()})
    for g in groups:
        b = int(rng.integers(w.B))
        log("  full-length group %d b=%d" % (g, b))
        _window_check(q, k, v, h, y, w, b, 0, L, g * w.group_size, (g + 1) * w.group_size)


def _assert_all_finite(y, what):
    """Every element of a NaN-prefilled output was written (scanned on the device)."""
    flat = y.view(-1)
    step = 1 << 28
    for i in range(0, flat.numel(), step):
        assert bool(torch.isfinite(flat[i:i + step]).all()), "%s: unwritten or non-finite output" % what


def _shards_match(w, q, k, v, h, y, rows):
    """Rows [s, s + rows) of each batch row (the last shard may be shorter),
    run through the history-prefix entry with the l_h - 1 rows before s as
    the prefix, give the same bits as the big call: spans start on chunk
    boundaries, so each output sums the same terms in the same order
    (StripedHyena 2 explainer, page "01. overview", section 5:
    point-to-point context parallelism).  A shard is a small grid with small
    (32-bit) offsets; for a 128-tap filter it takes the 8-wave kernel, whose
    Toeplitz fragments stay in registers, where the big call takes the
    16-wave one, so two kernels and two address ranges must agree."""
    assert rows % 64 == 0
    P = w.l_h - 1
    out = torch.empty((1, rows, w.D), dtype=y.dtype, device=y.device)
    for b in range(w.B):
        for s in range(0, w.L, rows):
            e = min(w.L, s + rows)
            sl = lambda a: a[b:b + 1, s:e]
            o = out[:, :e - s]
            if s == 0 or P == 0:
                hc.conv_fwd(sl(q), sl(k), sl(v), h, w.group_size, out=o)
            else:
                hc.conv_fwd(sl(q), sl(k), sl(v), h, w.group_size, out=o,
                            k_prev=k[b:b + 1, s - P:s], v_prev=v[b:b + 1, s - P:s])
            assert torch.equal(o, y[b:b + 1, s:e]), "%s: batch row %d, shard at row %d differs" % (w.name, b, s)


def _slab_width(B, L, D, gs, l_h):
    """Channels per workgroup of the plan: 256 (16 waves) or 128 (8 waves)."""
    span, wgs = hc.plan(B, L, D, gs, l_h)
    spans = B * -(-(-(-L // 64)) // span)
    assert wgs in (spans * -(-D // 256), spans * -(-D // 128))
    return 256 if wgs == spans * -(-D // 256) else 128


def test_mr_b4_sampled():
    w = WORKLOADS["mr_b4"]
    assert _slab_width(w.B, w.L, w.D, w.group_size, w.l_h) == 256
    assert _slab_width(1, 16384, w.D, w.group_size, w.l_h) == 128
    log("mr_b4: generate")
    q, k, v, h = make_inputs(w, DEV)
    y = run(q, k, v, h, w.group_size)
    _assert_all_finite(y, "mr_b4")
    log("mr_b4: 16384-row shards")
    _shards_match(w, q, k, v, h, y, 16384)
    _sampled_checks(w, q, k, v, h, y, n_groups=6, seed=4)


def test_wide_mr_ragged_partial_slab_sampled():
    """The 16-wave form of a 128-tap filter (taken from 1024 workgroups at
    8-chunk spans on) on a ragged length and a partial 256-channel slab."""
    w = dataclasses.replace(WORKLOADS["mr"], name="mr_wide_edge", B=2, L=262081, D=272)
    span, wgs = hc.plan(w.B, w.L, w.D, w.group_size, w.l_h)
    assert (span, wgs) == (8, 2 * 2 * 512)  # 2 slabs of 256 channels, 512 spans
    assert _slab_width(1, 16384, w.D, w.group_size, w.l_h) == 128
    log("mr_wide_edge: generate")
    q, k, v, h = make_inputs(w, DEV)
    y = run(q, k, v, h, w.group_size)
    _assert_all_finite(y, "mr_wide_edge")
    log("mr_wide_edge: 16384-row shards")
    _shards_match(w, q, k, v, h, y, 16384)
    _sampled_checks(w, q, k, v, h, y, n_groups=2, seed=6)


def test_long_stripe_sampled():
    """SE layer then MR layer at L = 2^20 (2^32 elements per tensor), one stream.

    Every output element is checked three ways: the whole NaN-prefilled
    output must be written; 16384-row shards, each run through the
    history-prefix entry with small (32-bit) offsets (for MR on the 8-wave
    kernel), must give the same bits; and windows (one straddling element
    2^31) and eight full-length groups (first, last, six seeded) are
    compared with the oracle.
    """
    outs = []
    for name in ("long_se", "long_mr"):
        w = WORKLOADS[name]
        log("%s: generate" % name)
        q, k, v, h = make_inputs(w, DEV)
        y = nan_like(q)
        hc.conv_fwd(q, k, v, h, w.group_size, out=y)
        outs.append((w, q, k, v, h, y))
    torch.cuda.synchronize()
    for w, q, k, v, h, y in outs:
        log("%s: whole-output scan" % w.name)
        _assert_all_finite(y, w.name)
        log("%s: 16384-row shards" % w.name)
        _shards_match(w, q, k, v, h, y, 16384)
        log("%s: sampled checks" % w.name)
        _sampled_checks(w, q, k, v, h, y, n_groups=6, seed=5)
        del q, k, v, h, y


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("l_h", [7, 33, 128])
def test_wider_group_matches_repeated_filters(dt, l_h):
    """group_size 32 is group_size 16 with each filter given to both of its
    16-channel tiles: a tile's Toeplitz products read only its own filter row,
    so y, dq, dk and dv agree bit for bit on any inputs (dh sums a group's
    channels and is not compared here)."""
    dtype = DTYPES[dt]
    B, L, D = 2, 1000, 256
    q, k, v, h32 = gaussian_inputs(B, L, D, 32, l_h, dtype, seed=500 + l_h)
    dy = gaussian_inputs(B, L, D, 32, 1, dtype, seed=600 + l_h)[0]
    h16 = torch.repeat_interleave(h32, 2, dim=0).contiguous()
    q, k, v, dy, h16, h32 = (t.to(DEV) for t in (q, k, v, dy, h16, h32))
    log("wider group %s l_h=%d: forward" % (dt, l_h))
    assert torch.equal(hc.conv_fwd(q, k, v, h32, 32), hc.conv_fwd(q, k, v, h16, 16))
    log("wider group %s l_h=%d: backward" % (dt, l_h))
    g32 = hc.conv_bwd(q, k, v, h32, dy, 32)
    g16 = hc.conv_bwd(q, k, v, h16, dy, 16)
    for name, a, b in zip(("dq", "dk", "dv"), g32[:3], g16[:3]):
        assert torch.equal(a, b), name
    assert bool(torch.isfinite(g32[3]).all())
