"""GPU parity of the long-filter backward (hyena_conv_bwd_long, FFT convolution).

Bars, per channel d of group g, batch row b and transform length N (fp32
transforms for both I/O types; x = k v and dz = dy q are exact in fp32 for
bf16 inputs), with e = (log2 N + 2) * 7 * 2^-24 and r = 2^-8 (bf16 output
rounding) or 2^-24 (fp32), the norm-wise error of an fp32 FFT convolution
carried through two forward transforms, the product and the inverse:

    dq: |err| <= r |ref| + |dy| * 3 e sqrt(N) ||h_g|| ||x_bd||
    dk: |err| <= r |ref| + |v|  * 3 e sqrt(N) ||h_g|| ||dz_bd||     (dv: |k|)
    dh: |err| <= 3 e sqrt(N) * sum_{b, d in g} ||dz_bd|| ||x_bd||

plus the gates max|err| <= 1e-2 max|ref| (bf16) or 1e-5 max|ref| (fp32) for
dq, dk, dv, and 1e-5 max|ref| for dh (fp32 output; an fp32 FFT correlation of
N(0, 1) sequences errs by about 2e-7 of the largest lag).
"""
import math

import pytest
import torch

import gated_convolution_sequence_amd as hc
from gpu_util import DEV, check_long_bwd, log, register_fed_forms, run_long_bwd as _run
from workloads import gaussian_inputs

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    hc.lib()
    yield
    torch.cuda.synchronize()


def _dy(B, L, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(B, L, D, generator=g).to(dtype)


SHAPES = [
    # B, L, D, group_size, l_h
    (1, 1, 2, 1, 1), (1, 6, 4, 2, 4), (1, 100, 8, 1, 100), (2, 257, 16, 16, 257),
    (1, 1000, 32, 2, 1000), (1, 1000, 32, 1, 37), (3, 777, 6, 3, 500), (1, 2048, 10, 5, 3000),
    (2, 3000, 128, 16, 128), (1, 4096, 64, 16, 4096), (1, 3000, 256, 256, 3000),
    (1, 8192, 16, 1, 8192),
    (1, 40000, 4, 2, 40000),     # N = 2^17: the three-level split
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_register_fed_and_lds_forms_agree(dt):
    """The backward's row, column and output passes with tiles of 4096
    values (register-fed first and last stages, D = 128) and with fewer
    channels (every stage through LDS, the first 32 channels alone): dq, dk,
    dv of those channels and dh of their groups agree within the FFT bars,
    and each call matches the oracle."""
    dtype = DTYPES[dt]
    B, L, l_h, gs = 2, 2000, 2000, 2
    wide, narrow = register_fed_forms(L, 128, gs, l_h), register_fed_forms(L, 32, gs, l_h)
    assert wide["rows"] and wide["bwd1"] and not narrow["rows"] and not narrow["bwd1"]
    q, k, v, h = gaussian_inputs(B, L, 128, gs, l_h, dtype, seed=67)
    dy = _dy(B, L, 128, dtype, seed=71)
    log("long bwd register-fed vs LDS forms %s" % dt)
    wide = [t.clone() for t in _run(*(t.to(DEV) for t in (q, k, v, h, dy)), gs)]
    sub = [t[..., :32].contiguous() for t in (q, k, v)]
    dys = dy[..., :32].contiguous()
    narrow = _run(*(t.to(DEV) for t in (*sub, h[:16].contiguous(), dys)), gs)
    for i, (a, b) in enumerate(zip(wide, narrow)):
        a = a[..., :32] if i < 3 else a[:16]
        scale = float(b.float().abs().max())
        tol = (1e-2 if dtype == torch.bfloat16 and i < 3 else 1e-5) * scale
        assert float((a.float() - b.float()).abs().max()) <= tol, "gradient %d" % i
    check_long_bwd(wide, q, k, v, h, dy, gs, dtype, "register-fed")
    check_long_bwd(narrow, *sub, h[:16].contiguous(), dys, gs, dtype, "LDS")


# every register-fed instance (64-, 128- and 256-point transforms), ragged
# last tiles, two batch rows, different radices for rows and columns
REGISTER_FED_SHAPES = [
    # B, L, D, group_size, l_h
    (2, 3000, 200, 2, 1000), (2, 5000, 136, 4, 3000), (1, 20000, 130, 2, 300), (1, 40000, 40, 8, 300),
    (1, 70000, 128, 2, 300),     # N = 2^17, three-level: 64-point columns and middle passes
    (1, 132000, 128, 2, 100),    # N = 2^18, three-level: 64 x 64 x 64, every pass register-fed
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h", REGISTER_FED_SHAPES)
def test_register_fed_shapes(dt, B, L, D, gs, l_h):
    forms = register_fed_forms(L, D, gs, l_h)
    assert forms["col1"] and forms["bwd1"] and (forms["rows"] or forms["mid"])
    log("long bwd register-fed %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=2 * L + D + gs)
    dy = _dy(B, L, D, dtype, seed=L + 11)
    got = _run(*(t.to(DEV) for t in (q, k, v, h, dy)), gs)
    rel = check_long_bwd(got, q, k, v, h, dy, gs, dtype, "long bwd register-fed")
    log("  rel err %s" % ", ".join("%s %.2e" % kv for kv in rel.items()))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_many_filters(dt):
    """Over 512 filters (G = 1040, group size 2) the filter pass transposes
    them first; all four gradients against the oracle."""
    dtype = DTYPES[dt]
    B, L, D, gs, l_h = 1, 1500, 2080, 2, 1500
    log("long bwd many filters %s" % dt)
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=89)
    dy = _dy(B, L, D, dtype, seed=97)
    got = _run(*(t.to(DEV) for t in (q, k, v, h, dy)), gs)
    check_long_bwd(got, q, k, v, h, dy, gs, dtype, "long bwd many filters")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h", SHAPES)
def test_long_backward_gaussian(dt, B, L, D, gs, l_h):
    log("long bwd %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=3 * L + l_h + gs)
    dy = _dy(B, L, D, dtype, seed=L + 5)
    got = _run(*(t.to(DEV) for t in (q, k, v, h, dy)), gs)
    rel = check_long_bwd(got, q, k, v, h, dy, gs, dtype, "long bwd")
    log("  rel err %s" % ", ".join("%s %.2e" % kv for kv in rel.items()))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_subsets_give_the_same_bits(dt):
    """dq alone, dk and dv alone, dh alone: the same bits as the full call."""
    dtype = DTYPES[dt]
    B, L, D, gs, l_h = 2, 1500, 24, 3, 900
    q, k, v, h = (t.to(DEV) for t in gaussian_inputs(B, L, D, gs, l_h, dtype, seed=77))
    dy = _dy(B, L, D, dtype, seed=78).to(DEV)
    full = [t.clone() for t in _run(q, k, v, h, dy, gs)]
    dq = _run(q, k, v, h, dy, gs, dkv=False, dh=False)
    dkv = _run(q, k, v, h, dy, gs, dq=False, dh=False)
    dh = _run(q, k, v, h, dy, gs, dq=False, dkv=False)
    assert dq[1] is None and dq[3] is None and dkv[0] is None and dh[0] is None
    assert torch.equal(dq[0], full[0])
    assert torch.equal(dkv[1], full[1]) and torch.equal(dkv[2], full[2])
    assert torch.equal(dh[3], full[3])
    again = _run(q, k, v, h, dy, gs)
    for a, b in zip(again, full):
        assert torch.equal(a, b)  # run to run


def test_matches_the_grouped_backward_for_short_filters():
    """l_h <= 128 with 16-channel groups: the FFT backward and the grouped
    kernels' backward (fp32) agree within their bars."""
    B, L, D, gs, l_h = 2, 5000, 256, 16, 128
    q, k, v, h = (t.to(DEV) for t in gaussian_inputs(B, L, D, gs, l_h, torch.float32, seed=15))
    dy = _dy(B, L, D, torch.float32, seed=16).to(DEV)
    log("fft bwd vs grouped bwd")
    fft = _run(q, k, v, h, dy, gs)
    direct = hc.conv_bwd(q, k, v, h, dy, gs)
    torch.cuda.synchronize()
    for a, b, name in zip(fft, direct, ("dq", "dk", "dv", "dh")):
        scale = float(b.abs().max())
        assert float((a - b).abs().max()) <= 2e-5 * scale, name


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_impulse_gradients_three_level(dt):
    """L = l_h = 2^19 (N = 2^20, three-level split), k = v = q = 1 and dy an
    impulse at t0 on every channel: dz is that impulse, so dx[t] = h[t0 - t]
    for t <= t0 and 0 after; dh[g, s] = group_size for s <= t0 (x = 1 at every
    row), 0 after; dq = h's prefix sums at t0 on row t0 only."""
    dtype = DTYPES[dt]
    B, L, D, gs = 1, 1 << 19, 4, 2
    t0 = 300000
    g = torch.Generator().manual_seed(19)
    h = (torch.randn(D // gs, L, generator=g) / math.sqrt(L)).to(dtype)
    ones = torch.ones(B, L, D, dtype=dtype)
    dy = torch.zeros(B, L, D, dtype=dtype)
    dy[0, t0, :] = 1.0
    log("impulse three-level %s" % dt)
    dq, dk, dv, dh = (t.float().cpu() for t in _run(*(t.to(DEV) for t in (ones, ones, ones, h, dy)), gs))
    hh = torch.repeat_interleave(h.float(), gs, dim=0)                # [D, L]
    expect_dx = torch.zeros(L, D)
    expect_dx[:t0 + 1, :] = hh[:, :t0 + 1].flip(1).T
    tol_x = (1e-2 if dtype == torch.bfloat16 else 1e-5) * float(expect_dx.abs().max())
    assert float((dk[0] - expect_dx).abs().max()) <= tol_x
    assert float((dv[0] - expect_dx).abs().max()) <= tol_x
    expect_dh = torch.zeros(D // gs, L)
    expect_dh[:, :t0 + 1] = gs
    assert float((dh - expect_dh).abs().max()) <= 1e-4 * gs
    expect_dq_t0 = hh[:, :t0 + 1].sum(dim=1)                          # z[t0] = sum_s h[s] x[t0 - s]
    scale = float(expect_dq_t0.abs().max())
    assert float((dq[0, t0] - expect_dq_t0).abs().max()) <= (1e-2 if dtype == torch.bfloat16 else 1e-4) * scale
    dq[0, t0] = 0
    assert float(dq.abs().max()) == 0.0   # dy is zero elsewhere


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,gs,l_h", [(0, 100, 2, 300), (2, 0, 1, 7)])
def test_backward_without_rows_zeroes_dh(dt, B, L, gs, l_h):
    """No rows: dh is written with zeros (the caller's buffer starts as NaN
    here), by a kernel; no workspace is needed."""
    dtype, D = DTYPES[dt], 8
    log("long bwd no rows %s B=%d L=%d" % (dt, B, L))
    buf = torch.zeros(64, dtype=dtype, device=DEV)  # q, k, v, dy: no rows are read
    h = torch.ones(D // gs, l_h, dtype=dtype, device=DEV)
    dh = torch.full((D // gs, l_h), float("nan"), dtype=torch.float32, device=DEV)
    code = hc.DTYPE_BF16 if dt == "bf16" else hc.DTYPE_F32
    assert hc.bwd_long_workspace_bytes(B, L, D, gs, l_h, code) == 0
    p = buf.data_ptr()
    st = hc.lib().hyena_conv_bwd_long(p, p, p, h.data_ptr(), p, B, L, D, gs, l_h, None, None, None,
                                      dh.data_ptr(), code, None, 0, torch.cuda.current_stream(DEV).cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(dh, torch.zeros_like(dh))


def test_autograd_wrapper_matches_the_entry_point():
    B, L, D, gs, l_h = 2, 700, 12, 3, 900
    q, k, v, h = (t.to(DEV) for t in gaussian_inputs(B, L, D, gs, l_h, torch.float32, seed=31))
    dy = _dy(B, L, D, torch.float32, seed=32).to(DEV)
    leaves = [t.clone().requires_grad_(True) for t in (q, k, v, h)]
    y = hc.HyenaConvLong.apply(*leaves, gs)
    y.backward(dy)
    want = hc.conv_bwd_long(q, k, v, h, dy, gs)
    torch.cuda.synchronize()
    assert torch.equal(y, hc.conv_fwd_long(q, k, v, h, gs))
    for leaf, w in zip(leaves, want):
        assert torch.equal(leaf.grad, w)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("L,D,gs,l_h", [(1000, 64, 16, 1000), (3000, 48, 3, 700), (300, 8, 1, 5000)])
def test_kept_filter_spectra_give_the_same_bits(dt, L, D, gs, l_h):
    """hyena_conv_bwd_long_ex with reuse_spectra: a forward on the backward's
    workspace leaves the filter spectra there; a backward that reuses them
    (h passed as NULL, the rest of the workspace filled with NaN) equals one
    that computes them, bit for bit."""
    dtype = DTYPES[dt]
    log("long bwd kept spectra %s L=%d D=%d gs=%d l_h=%d" % (dt, L, D, gs, l_h))
    q, k, v, h = (t.to(DEV) for t in gaussian_inputs(2, L, D, gs, l_h, dtype, seed=L + 3))
    dy = _dy(2, L, D, dtype, seed=L + 4).to(DEV)
    code = hc.DTYPE_BF16 if dtype == torch.bfloat16 else hc.DTYPE_F32
    n = hc.bwd_long_workspace_bytes(2, L, D, gs, l_h, code)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    hc.conv_fwd_long(q, k, v, h, gs, workspace=ws)
    N = 1 << max(2, (L + min(l_h, L) - 2).bit_length())
    G = D // gs
    spectra = 8 * N * (G + (G & 1))
    ws[spectra:].view(torch.float32).fill_(float("nan"))
    outs = [torch.empty_like(q) for _ in range(3)] + [torch.empty(G, l_h, device=DEV)]
    st = hc.lib().hyena_conv_bwd_long_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), None, dy.data_ptr(), 2, L, D, gs,
                                         l_h, *[o.data_ptr() for o in outs], code, ws.data_ptr(), n, 1,
                                         torch.cuda.current_stream().cuda_stream)
    assert st == 0, hc.strerror(st)
    fresh = hc.conv_bwd_long(q, k, v, h, dy, gs)
    torch.cuda.synchronize()
    for a, b in zip(outs, fresh):
        assert torch.equal(a, b)


def test_hyena_conv_routes_long_filters_to_the_fft_path():
    """HyenaConv with a filter over 128 taps runs the FFT path: the same
    output and gradients, bit for bit, as HyenaConvLong."""
    B, L, D, gs, l_h = 1, 600, 32, 4, 700
    q, k, v, h = (t.to(DEV) for t in gaussian_inputs(B, L, D, gs, l_h, torch.bfloat16, seed=71))
    dy = _dy(B, L, D, torch.bfloat16, seed=72).to(DEV)
    grads = []
    for fn in (hc.HyenaConv, hc.HyenaConvLong):
        leaves = [t.clone().requires_grad_(True) for t in (q, k, v, h)]
        y = fn.apply(*leaves, gs)
        y.backward(dy)
        grads.append([y.detach()] + [t.grad for t in leaves])
    torch.cuda.synchronize()
    for a, b in zip(*grads):
        assert torch.equal(a, b)
