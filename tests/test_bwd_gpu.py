"""GPU parity of the backward (hyena_conv_bwd) against the fp64 backward oracle.

The bar, per gradient, from the rounding the library does (dz = dy q and
x = k v rounded once to bf16 as matrix-core operands, fp32 sums, one output
rounding), with env the same gradient computed on magnitudes:
  dq, dk, dv (bf16): |e| <= 2^-8 |ref| + (2^-8 (1 + 2^-8) + l_h 2^-23) env
  dq, dk, dv (fp32): |e| <= 2^-24 |ref| + (l_h + 4) 2^-23 env
  dh (fp32 output):  |e| <= (u_in + (R + 256) 2^-24) env,  u_in = 2^-7 + 2^-14
                     (bf16 inputs) or 4 * 2^-24 (fp32), R = partial rows summed
plus the gate max|e| <= 1e-2 max|ref| (bf16) / 1e-5 max|ref| (fp32).
Integer inputs are exact in every intermediate, so they must match bitwise.
"""
import numpy as np
import pytest
import torch

import gated_convolution_sequence_amd as hc
import oracle
from gpu_util import DEV, bwd_refs, bwd_rows, check, check_bwd, check_dh, log, to_np
from workloads import WORKLOADS, gaussian_inputs, integer_inputs, make_inputs, normal_activation

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    hc.lib()


def _bwd_gpu(q, k, v, h, dy, gs):
    out = hc.conv_bwd(q, k, v, h, dy, gs)
    torch.cuda.synchronize()
    return out


_refs = bwd_refs
_check_dh = check_dh
_check_all = check_bwd
_rows = bwd_rows


BWD_SHAPES = [
    # B, L, D, group_size, l_h
    (1, 1, 16, 16, 1), (1, 6, 16, 16, 4), (1, 63, 32, 16, 7), (2, 130, 48, 16, 33),
    (1, 700, 64, 32, 128), (3, 257, 128, 16, 65), (1, 1000, 96, 48, 97), (1, 2048, 256, 16, 128),
    (2, 515, 208, 16, 2),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h", BWD_SHAPES)
def test_backward_gaussian(dt, B, L, D, gs, l_h):
    log("bwd %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=7 * L + l_h)
    dy = normal_activation((B, L, D), dtype, "cpu", seed=L + 1)
    dev = [t.to(DEV) for t in (q, k, v, h, dy)]
    grads = _bwd_gpu(*dev, gs)
    ref, env = _refs(q, k, v, h, dy, gs)
    _check_all(grads, ref, env, l_h, dtype, _rows(B, L, D, gs, l_h, dtype), "bwd")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h", [(1, 6, 16, 16, 4), (2, 777, 96, 32, 7),
                                          (1, 1000, 64, 16, 128), (3, 130, 16, 16, 66)])
def test_backward_integer_inputs_bitwise(dt, B, L, D, gs, l_h):
    log("bwd integer %s B=%d L=%d D=%d l_h=%d" % (dt, B, L, D, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = integer_inputs(B, L, D, gs, l_h, dtype, seed=L + 3)
    dy = integer_inputs(B, L, D, gs, 1, dtype, seed=L + 4)[0]
    grads = _bwd_gpu(*[t.to(DEV) for t in (q, k, v, h, dy)], gs)
    ref = oracle.conv_bwd_ref(*[to_np(t) for t in (q, k, v, h, dy)], gs)
    for name, g, r in zip(("dq", "dk", "dv", "dh"), grads, ref):
        assert np.array_equal(to_np(g), r), name


SUBSETS = [(True, False, False), (False, True, False), (False, False, True),
           (True, False, True), (True, True, False), (False, True, True)]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h", [(1, 6, 16, 16, 4), (2, 777, 96, 32, 7), (3, 257, 128, 16, 65),
                                          (1, 1000, 96, 48, 97), (1, 2048, 256, 16, 128),
                                          (2, 768, 96, 32, 7), (3, 320, 48, 16, 65), (1, 1024, 128, 16, 128),
                                          (1, 96, 32, 16, 1)])
def test_output_subsets_match_the_full_call(dt, B, L, D, gs, l_h):
    """Which gradients are requested decides which kernels run: in bf16 all
    four are one pass walked backwards in time; dq with dh is one pass in
    time order; dk and dv alone are the forward kernel walked backwards; dq
    alone is the forward kernel; dh alone is its own pass.  fp32 always takes
    the separate kernels, so every gradient has the same bits on every route.
    In bf16, dk and dv of the one pass equal the backwards forward kernel's
    bit for bit (the same walk).  dq sums each 32-row block of x as one
    matrix-core step; the backwards walk aligns its blocks to the sequence's
    end and the time-order routes to its start, so dq has the same bits when
    L is a multiple of 32.  dh sums the spans' chunks in the opposite order.
    Where the order differs, the other route's result is held to the oracle
    bound as well."""
    dtype = DTYPES[dt]
    log("bwd subsets %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=B + L + l_h)
    dy = normal_activation((B, L, D), dtype, "cpu", seed=L + 5)
    dev = [t.to(DEV) for t in (q, k, v, h, dy)]
    full = hc.conv_bwd(*dev, gs)
    oracle_ref = []

    def refs():
        if not oracle_ref:
            oracle_ref.append(_refs(q, k, v, h, dy, gs))
        return oracle_ref[0]

    def same_bits(name):
        if dt == "f32" or name in ("dk", "dv"):
            return True
        return name == "dq" and L % 32 == 0

    for need in SUBSETS:
        part = hc.conv_bwd(*dev, gs, need_dq=need[0], need_dkv=need[1], need_dh=need[2])
        torch.cuda.synchronize()
        wanted = (need[0], need[1], need[1], need[2])
        for j, (name, want, f, g) in enumerate(zip(("dq", "dk", "dv", "dh"), wanted, full, part)):
            assert (g is not None) == want, (name, need)
            if not want:
                continue
            if same_bits(name):
                assert torch.equal(f, g), (name, need)
            elif name == "dh":
                ref, env = refs()
                _check_dh(g, ref[3], env[3], dtype, _rows(B, L, D, gs, l_h, dtype), "subset %s" % (need,))
            else:
                ref, env = refs()
                check(to_np(g), ref[j], env[j], l_h, dtype, "subset %s %s" % (need, name))


def test_backward_deterministic():
    q, k, v, h = gaussian_inputs(2, 1500, 256, 16, 128, torch.bfloat16, seed=21)
    dy = normal_activation((2, 1500, 256), torch.bfloat16, "cpu", seed=22)
    dev = [t.to(DEV) for t in (q, k, v, h, dy)]
    a = _bwd_gpu(*dev, 16)
    b = _bwd_gpu(*dev, 16)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_autograd_function_matches_the_oracle():
    log("autograd wrapper")
    B, L, D, gs, l_h = 1, 500, 64, 16, 100
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, torch.bfloat16, seed=31)
    dy = normal_activation((B, L, D), torch.bfloat16, "cpu", seed=32)
    tq, tk, tv, th = (t.to(DEV).requires_grad_(True) for t in (q, k, v, h))
    y = hc.HyenaConv.apply(tq, tk, tv, th, gs)
    y.backward(dy.to(DEV))
    ref, env = _refs(q, k, v, h, dy, gs)
    for name, t, r, e in zip(("dq", "dk", "dv"), (tq, tk, tv), ref, env):
        check(to_np(t.grad), r, e, l_h, torch.bfloat16, "autograd " + name)
    # dh comes back in h's dtype (bf16): one more rounding
    got = to_np(th.grad)
    assert np.max(np.abs(got - ref[3])) <= 1e-2 * np.max(np.abs(ref[3]))


@pytest.mark.parametrize("name", ["se", "mr"])
def test_backward_full_workload(name):
    w = WORKLOADS[name]
    log("bwd %s full: generate" % name)
    q, k, v, h = make_inputs(w, DEV)
    dy = normal_activation((w.B, w.L, w.D), w.torch_dtype, DEV, seed=w.seed + 9)
    grads = _bwd_gpu(q, k, v, h, dy, w.group_size)
    log("bwd %s full: oracle" % name)
    ref, env = _refs(q, k, v, h, dy, w.group_size)
    _check_all(grads, ref, env, w.l_h, w.torch_dtype, _rows(w.B, w.L, w.D, w.group_size, w.l_h,
                                                            w.torch_dtype), name)


def test_backward_mr_b4_sampled():
    """dq, dk, dv on exact windows; dh of whole groups (it sums every row)."""
    w = WORKLOADS["mr_b4"]
    log("bwd mr_b4: generate")
    q, k, v, h = make_inputs(w, DEV)
    dy = normal_activation((w.B, w.L, w.D), w.torch_dtype, DEV, seed=w.seed + 9)
    dq, dk, dv, dh = _bwd_gpu(q, k, v, h, dy, w.group_size)
    gs, lh = w.group_size, w.l_h
    for b, t0, t1 in ((0, 0, 256), (3, w.L // 2 - 100, w.L // 2 + 37), (3, w.L - 256, w.L)):
        log("  window b=%d [%d,%d)" % (b, t0, t1))
        s, e = max(0, t0 - (lh - 1)), min(w.L, t1 + lh - 1)  # past for dq, future for dk, dv
        sl = lambda a: a[b:b + 1, s:e]
        ref, env = _refs(sl(q), sl(k), sl(v), h, sl(dy), gs)
        o0, o1 = t0 - s, t1 - s
        for nm, g, r, en in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, env):
            check(to_np(g[b:b + 1, t0:t1]), r[:, o0:o1], en[:, o0:o1], lh, w.torch_dtype, "mr_b4 " + nm)
    for g in (0, 77, w.G - 1):
        log("  dh group %d" % g)
        c = slice(g * gs, (g + 1) * gs)
        ref, env = _refs(q[:, :, c].contiguous(), k[:, :, c].contiguous(), v[:, :, c].contiguous(),
                         h[g:g + 1], dy[:, :, c].contiguous(), gs)
        _check_dh(dh[g:g + 1], ref[3], env[3], w.torch_dtype,
                  _rows(w.B, w.L, w.D, gs, lh, w.torch_dtype), "mr_b4 dh")


# Off the 16-channel tile with at most 8 taps: the direct kernels (dq with
# the partial dh sums in one walk, dx walked backwards in time with two
# gates, a reduction per group).  B, L, D, group_size, l_h: lengths below the
# filter and across span seams, partial 256-channel slabs, each compiled tap
# count (1, 2, 4, 8) and the lengths padded up to them.
BWD_DIRECT_SHAPES = [
    (1, 1, 8, 1, 1), (1, 6, 8, 1, 4), (2, 130, 264, 3, 7), (1, 700, 40, 5, 8),
    (3, 257, 96, 8, 2), (1, 2048, 512, 1, 7), (2, 515, 24, 2, 6),
]


def _direct_rows(B, L, D, gs, l_h, dtype):
    """Partial sums behind each dh value: one per span, batch row and channel of the group."""
    code = hc.DTYPE_BF16 if dtype == torch.bfloat16 else hc.DTYPE_F32
    return max(1, hc.bwd_workspace_bytes(B, L, D, gs, l_h, code) // (D * l_h * 4)) * gs


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h", BWD_DIRECT_SHAPES)
def test_backward_off_tile_short_filters_gaussian(dt, B, L, D, gs, l_h):
    log("bwd direct %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=11 * L + l_h + gs)
    dy = normal_activation((B, L, D), dtype, "cpu", seed=L + 9)
    grads = _bwd_gpu(*[t.to(DEV) for t in (q, k, v, h, dy)], gs)
    ref, env = _refs(q, k, v, h, dy, gs)
    _check_all(grads, ref, env, l_h, dtype, _direct_rows(B, L, D, gs, l_h, dtype), "bwd direct")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h", [(1, 6, 8, 1, 4), (2, 777, 96, 3, 7), (1, 300, 264, 8, 8)])
def test_backward_off_tile_integer_inputs_bitwise(dt, B, L, D, gs, l_h):
    log("bwd direct integer %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = integer_inputs(B, L, D, gs, l_h, dtype, seed=L + 13)
    dy = integer_inputs(B, L, D, gs, 1, dtype, seed=L + 14)[0]
    grads = _bwd_gpu(*[t.to(DEV) for t in (q, k, v, h, dy)], gs)
    ref = oracle.conv_bwd_ref(*[to_np(t) for t in (q, k, v, h, dy)], gs)
    for name, g, r in zip(("dq", "dk", "dv", "dh"), grads, ref):
        assert np.array_equal(to_np(g), r), name


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_off_tile_subsets_match_the_full_call(dt):
    """dq alone is the direct forward with dy as the gate, which sums as the
    one walk does; dh alone and dk, dv alone are the same kernels as in the
    full call: every gradient has the same bits on every route."""
    dtype = DTYPES[dt]
    B, L, D, gs, l_h = 2, 1000, 264, 3, 7
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=41)
    dy = normal_activation((B, L, D), dtype, "cpu", seed=42)
    dev = [t.to(DEV) for t in (q, k, v, h, dy)]
    full = hc.conv_bwd(*dev, gs)
    for need in SUBSETS:
        part = hc.conv_bwd(*dev, gs, need_dq=need[0], need_dkv=need[1], need_dh=need[2])
        torch.cuda.synchronize()
        wanted = (need[0], need[1], need[1], need[2])
        for name, want, f, g in zip(("dq", "dk", "dv", "dh"), wanted, full, part):
            assert (g is not None) == want, (name, need)
            if want:
                assert torch.equal(f, g), (name, need)


# Off the 16-channel tile with more than 8 taps: dq and dk, dv from the
# chunk-direction kernel (forward, and walked backwards in time with two
# gates), dh from per-channel lag products and the per-group reduction.
# B, L, D, group_size, l_h: group sizes 1, 3 and 8 and filters of 9, 65 and
# 128 taps among them, lengths across 64-row blocks, 256-row chunk-direction
# blocks and 1024-row filter-gradient spans, partial channel slabs.
BWD_CD_SHAPES = [
    (1, 300, 64, 1, 9), (2, 1000, 72, 3, 65), (1, 700, 128, 8, 128), (1, 2100, 40, 5, 100),
    (3, 64, 24, 3, 33), (1, 1, 16, 8, 9), (2, 130, 48, 1, 128), (1, 1030, 264, 8, 65),
    (1, 500, 72, 3, 9), (2, 257, 64, 1, 65), (1, 1100, 24, 3, 128),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h", BWD_CD_SHAPES)
def test_backward_off_tile_long_filters_gaussian(dt, B, L, D, gs, l_h):
    log("bwd cd %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=13 * L + l_h + gs)
    dy = normal_activation((B, L, D), dtype, "cpu", seed=L + 19)
    grads = _bwd_gpu(*[t.to(DEV) for t in (q, k, v, h, dy)], gs)
    ref, env = _refs(q, k, v, h, dy, gs)
    _check_all(grads, ref, env, l_h, dtype, _direct_rows(B, L, D, gs, l_h, dtype), "bwd cd")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h", [(1, 300, 64, 1, 9), (2, 777, 96, 3, 65), (1, 600, 264, 8, 128)])
def test_backward_off_tile_long_filters_integer_bitwise(dt, B, L, D, gs, l_h):
    log("bwd cd integer %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = integer_inputs(B, L, D, gs, l_h, dtype, seed=L + 23)
    dy = integer_inputs(B, L, D, gs, 1, dtype, seed=L + 24)[0]
    grads = _bwd_gpu(*[t.to(DEV) for t in (q, k, v, h, dy)], gs)
    ref = oracle.conv_bwd_ref(*[to_np(t) for t in (q, k, v, h, dy)], gs)
    for name, g, r in zip(("dq", "dk", "dv", "dh"), grads, ref):
        assert np.array_equal(to_np(g), r), name


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_off_tile_long_filters_subsets_and_determinism(dt):
    """Each gradient has one kernel whatever else is requested, so every
    subset gives the full call's bits; a second call gives the same bits."""
    dtype = DTYPES[dt]
    B, L, D, gs, l_h = 2, 1300, 72, 3, 100
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=43)
    dy = normal_activation((B, L, D), dtype, "cpu", seed=44)
    dev = [t.to(DEV) for t in (q, k, v, h, dy)]
    full = hc.conv_bwd(*dev, gs)
    again = hc.conv_bwd(*dev, gs)
    torch.cuda.synchronize()
    for f, g in zip(full, again):
        assert torch.equal(f, g)
    for need in SUBSETS:
        part = hc.conv_bwd(*dev, gs, need_dq=need[0], need_dkv=need[1], need_dh=need[2])
        torch.cuda.synchronize()
        wanted = (need[0], need[1], need[1], need[2])
        for name, want, f, g in zip(("dq", "dk", "dv", "dh"), wanted, full, part):
            assert (g is not None) == want, (name, need)
            if want:
                assert torch.equal(f, g), (name, need)


def test_backward_off_tile_one_filter_per_channel_medium():
    """group_size 1, l_h = 128 (the MR filter length), B=1, L=2048, D=512 bf16."""
    B, L, D, gs, l_h = 1, 2048, 512, 1, 128
    log("bwd cd medium")
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, torch.bfloat16, seed=51)
    dy = normal_activation((B, L, D), torch.bfloat16, "cpu", seed=52)
    grads = _bwd_gpu(*[t.to(DEV) for t in (q, k, v, h, dy)], gs)
    ref, env = _refs(q, k, v, h, dy, gs)
    _check_all(grads, ref, env, l_h, torch.bfloat16, _direct_rows(B, L, D, gs, l_h, torch.bfloat16), "bwd cd medium")



@pytest.mark.parametrize("name", ["se", "mr"])
def test_backward_one_filter_per_channel_full_sampled(name):
    """The layer at its full size (B=1, L=8192, D=4096) with one filter per
    channel (each channel its group's taps, as the benchmark times it): SE
    through the direct kernels, MR through the chunk-direction passes and
    the matrix-core lag products.  Every output element must be finite, and
    all four gradients of eight whole channels (first, last and six seeded)
    are compared with the oracle run on those channels alone (with one
    filter per channel the operator is separable by channel)."""
    w = WORKLOADS[name]
    log("bwd %s group_size 1 full: generate" % name)
    q, k, v, h = make_inputs(w, DEV)
    h1 = torch.repeat_interleave(h, w.group_size, dim=0).contiguous()
    dy = normal_activation((w.B, w.L, w.D), w.torch_dtype, DEV, seed=w.seed + 9)
    dq, dk, dv, dh = _bwd_gpu(q, k, v, h1, dy, 1)
    for nm, g in (("dq", dq), ("dk", dk), ("dv", dv), ("dh", dh)):
        assert bool(torch.isfinite(g).all()), "%s %s: non-finite output" % (name, nm)
    rows = _direct_rows(w.B, w.L, w.D, 1, w.l_h, w.torch_dtype)
    rng = np.random.default_rng(w.seed)
    chans = sorted({0, w.D - 1, *rng.choice(w.D, size=6, replace=False).tolist()})
    for c in chans:
        log("  channel %d" % c)
        sl = lambda a: a[:, :, c:c + 1].contiguous()
        ref, env = _refs(sl(q), sl(k), sl(v), h1[c:c + 1], sl(dy), 1)
        for nm, g, r, en in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, env):
            check(to_np(sl(g)), r, en, w.l_h, w.torch_dtype, "%s gs1 %s channel %d" % (name, nm, c))
        check_dh(dh[c:c + 1], ref[3], env[3], w.torch_dtype, rows, "%s gs1 dh channel %d" % (name, c))

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,gs,l_h", [(0, 64, 16, 7), (2, 0, 16, 128), (1, 0, 1, 7)])
def test_backward_without_rows_zeroes_dh(dt, B, L, gs, l_h):
    """No rows: dq, dk, dv are empty and dh is written with zeros (the caller's
    buffer starts as NaN here), by a kernel."""
    dtype, D = DTYPES[dt], 64
    log("no rows %s B=%d L=%d gs=%d l_h=%d" % (dt, B, L, gs, l_h))
    buf = torch.zeros(64, dtype=dtype, device=DEV)  # q, k, v, dy: no rows are read
    h = torch.ones(D // gs, l_h, dtype=dtype, device=DEV)
    dh = torch.full((D // gs, l_h), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    code = hc.DTYPE_BF16 if dt == "bf16" else hc.DTYPE_F32
    p = buf.data_ptr()
    st = hc.lib().hyena_conv_bwd(p, p, p, h.data_ptr(), p, B, L, D, gs, l_h, None, None, None,
                                 dh.data_ptr(), ws.data_ptr(), 16, code,
                                 torch.cuda.current_stream(DEV).cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(dh, torch.zeros_like(dh))
