"""GPU parity of the long-filter forward (hyena_conv_fwd_long, FFT convolution).

The FFT path's rounding error is not local: every output row mixes every
input row through the transforms.  The bar, per channel d of group g and
transform length N (fp32 transforms for both I/O types; x = k v is exact in
fp32 for bf16 inputs):

    |y - y_ref| <= r |y_ref| + |q| * 3 e sqrt(N) ||h_g||_2 ||x_d||_2,
    e = (log2 N + 2) * 7 * 2^-24,

with r = 2^-8 (bf16 output rounding) or 2^-24 (fp32).  That is the norm-wise
error of a radix-2 FFT (per level at most about 7 units of rounding with
accurate twiddles; log2 N levels plus the two twiddle passes of the
four-step split), carried through the forward transforms of x and h, the
product and the inverse transform.  It is loose; the spec gate
max|y - y_ref| <= 1e-2 max|y_ref| (bf16) or 1e-5 max|y_ref| (fp32) is the
tight check, and is applied to every case.
"""
import math

import numpy as np
import pytest
import torch

import gated_convolution_sequence_amd as hc
import oracle
from gpu_util import DEV, check_long, log, register_fed_forms, run_long, to_np
from workloads import WORKLOADS, gaussian_inputs, make_inputs

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    hc.lib()
    yield
    torch.cuda.synchronize()


SHAPES = [
    # B, L, D, group_size, l_h
    (1, 1, 2, 1, 1), (1, 6, 4, 2, 4), (1, 100, 8, 1, 100), (2, 257, 16, 16, 257),
    (1, 1000, 32, 2, 1000), (1, 1000, 32, 1, 37), (1, 4096, 64, 16, 4096),
    (3, 777, 6, 3, 500), (1, 2048, 10, 5, 3000), (2, 3000, 128, 16, 128),
    (1, 8192, 256, 1, 8192), (1, 65536, 8, 8, 65536),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h", SHAPES)
def test_long_filter_gaussian(dt, B, L, D, gs, l_h):
    log("long %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=L + 7 * l_h + gs)
    y = run_long(q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV), gs)
    rel = check_long(y, q, k, v, h, gs, dtype, "long")
    log("  rel err %.3e" % rel)


@pytest.mark.parametrize("t0", [0, 1, 63, 64, 1000, 4095])
def test_impulse_reproduces_the_filter(t0):
    """x = delta at t0, q = 1: z[t0 + s] = h[s] up to fp32 transform rounding."""
    B, L, D, gs, l_h = 1, 4096, 4, 1, 4096
    rng = np.random.default_rng(t0)
    h = torch.tensor(rng.standard_normal((D, l_h)) / math.sqrt(l_h), dtype=torch.float32)
    v = torch.zeros(B, L, D)
    v[0, t0, :] = 1.0
    ones = torch.ones_like(v)
    log("impulse t0=%d" % t0)
    y = to_np(run_long(ones.to(DEV), ones.to(DEV), v.to(DEV), h.to(DEV), gs))
    expect = np.zeros((L, D))
    expect[t0:, :] = to_np(h).T[:L - t0]
    assert np.max(np.abs(y[0] - expect)) <= 1e-5 * np.max(np.abs(expect))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_largest_transform_impulse(dt):
    """L = l_h = 2^21 (N = 2^22, the largest transform): an impulse at t0 on
    every channel returns the filter shifted by t0, checked on all rows."""
    dtype = DTYPES[dt]
    B, L, D, gs = 1, 1 << 21, 4, 2
    t0 = 12345
    g = torch.Generator().manual_seed(21)
    h = (torch.randn(D // gs, L, generator=g) / math.sqrt(L)).to(dtype)
    v = torch.zeros(B, L, D, dtype=dtype)
    v[0, t0, :] = 1.0
    ones = torch.ones_like(v)
    log("largest transform %s" % dt)
    y = run_long(ones.to(DEV), ones.to(DEV), v.to(DEV), h.to(DEV), gs)[0].float().cpu()
    expect = torch.zeros(L, D)
    expect[t0:, :] = torch.repeat_interleave(h.float(), gs, dim=0).T[:L - t0]
    scale = float(expect.abs().max())
    tol = (1e-2 if dtype == torch.bfloat16 else 1e-5) * scale
    assert float((y - expect).abs().max()) <= tol
    assert float(y[:t0].abs().max()) <= tol  # nothing before the impulse


def test_matches_the_direct_kernel_for_short_filters():
    """l_h <= 128: the FFT path and the direct grouped kernel agree within their bars."""
    B, L, D, gs, l_h = 2, 5000, 256, 16, 128
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, torch.float32, seed=5)
    dev = [t.to(DEV) for t in (q, k, v, h)]
    log("fft vs direct")
    y_fft = run_long(*dev, gs)
    y_dir = hc.conv_fwd(*dev, gs)
    torch.cuda.synchronize()
    scale = float(y_dir.abs().max())
    assert float((y_fft - y_dir).abs().max()) <= 2e-5 * scale


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_single_and_paired_column_kernels_agree(dt):
    """An even group size runs the single-column kernel, group size 1 the
    paired one (the partner column separates the two channels' spectra).
    With each channel given its group's filter the two compute the same
    convolution; they agree within the FFT bar, and each matches the oracle."""
    dtype = DTYPES[dt]
    B, L, D, l_h = 2, 3000, 64, 3000
    q, k, v, h2 = gaussian_inputs(B, L, D, 2, l_h, dtype, seed=41)
    h1 = torch.repeat_interleave(h2, 2, dim=0).contiguous()
    dev = [t.to(DEV) for t in (q, k, v)]
    log("single vs paired columns %s" % dt)
    y2 = run_long(*dev, h2.to(DEV), 2).clone()
    y1 = run_long(*dev, h1.to(DEV), 1)
    scale = float(y1.float().abs().max())
    tol = (1e-2 if dtype == torch.bfloat16 else 1e-5) * scale
    assert float((y1.float() - y2.float()).abs().max()) <= tol
    check_long(y2, q, k, v, h2, 2, dtype, "single-column")
    check_long(y1, q, k, v, h1, 1, dtype, "paired")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_register_fed_and_lds_forms_agree(dt):
    """With tiles of 4096 values the row, single-column and output kernels
    keep a transform's first and last stages in registers; with fewer
    channels they run every stage through LDS.  Channels do not interact, so
    the first 64 channels of a D = 128 call (register-fed) and a D = 64 call
    on them (LDS) compute the same convolution: they agree within the FFT
    bar, and each matches the oracle."""
    dtype = DTYPES[dt]
    B, L, l_h, gs = 2, 2000, 2000, 2
    wide, narrow = register_fed_forms(L, 128, gs, l_h), register_fed_forms(L, 64, gs, l_h)
    assert wide["rows"] and wide["col1"] and not narrow["rows"] and not narrow["col1"]
    q, k, v, h = gaussian_inputs(B, L, 128, gs, l_h, dtype, seed=61)
    log("register-fed vs LDS forms %s" % dt)
    yw = run_long(q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV), gs).clone()
    sub = [t[..., :64].contiguous() for t in (q, k, v)]
    yn = run_long(*(t.to(DEV) for t in sub), h[:32].contiguous().to(DEV), gs)
    scale = float(yn.float().abs().max())
    tol = (1e-2 if dtype == torch.bfloat16 else 1e-5) * scale
    assert float((yw[..., :64].float() - yn.float()).abs().max()) <= tol
    check_long(yw, q, k, v, h, gs, dtype, "register-fed")
    check_long(yn, *sub, h[:32].contiguous(), gs, dtype, "LDS")


# shapes that reach every register-fed instance (last radix 4, 8 and 16:
# 64-, 128- and 256-point transforms), with a ragged last pair tile, two
# batch rows and a split with different radices for rows and columns
REGISTER_FED_SHAPES = [
    # B, L, D, group_size, l_h
    (2, 3000, 200, 2, 1000),     # N = 2^12: 64 x 64, tiles of 64 pairs (64 + 36)
    (2, 5000, 136, 4, 3000),     # N = 2^13: 128 columns, 64-point rows, 68 pairs
    (1, 20000, 130, 2, 300),     # N = 2^15: 256 columns, 128-point rows, 65 pairs
    (1, 40000, 40, 8, 300),      # N = 2^16: 256 x 256, tiles of 16 pairs (16 + 4)
    (1, 70000, 128, 2, 300),     # N = 2^17, three-level: 64-point columns and middle passes
    (1, 132000, 128, 2, 100),    # N = 2^18, three-level: 64 x 64 x 64, every pass register-fed
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,D,gs,l_h", REGISTER_FED_SHAPES)
def test_register_fed_shapes(dt, B, L, D, gs, l_h):
    forms = register_fed_forms(L, D, gs, l_h)
    assert forms["col1"] and (forms["rows"] or forms["mid"])
    log("long register-fed %s B=%d L=%d D=%d gs=%d l_h=%d" % (dt, B, L, D, gs, l_h))
    dtype = DTYPES[dt]
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=L + D + gs)
    y = run_long(q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV), gs)
    rel = check_long(y, q, k, v, h, gs, dtype, "long register-fed")
    log("  rel err %.3e" % rel)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_many_filters(dt):
    """Over 512 filters the filter pass first transposes them to fp32
    [taps][G'] (fewer are read from h [G][l_h] directly): G = 1024 here, one
    filter per channel, against the oracle."""
    dtype = DTYPES[dt]
    B, L, D, gs, l_h = 1, 2000, 1024, 1, 2000
    log("long many filters %s" % dt)
    q, k, v, h = gaussian_inputs(B, L, D, gs, l_h, dtype, seed=83)
    y = run_long(q.to(DEV), k.to(DEV), v.to(DEV), h.to(DEV), gs)
    check_long(y, q, k, v, h, gs, dtype, "many filters")


def test_deterministic_and_workspace_reuse():
    B, L, D, gs, l_h = 1, 3000, 64, 2, 3000
    q, k, v, h = (t.to(DEV) for t in gaussian_inputs(B, L, D, gs, l_h, torch.bfloat16, seed=9))
    ws = torch.empty(hc.long_workspace_bytes(B, L, D, gs, l_h), dtype=torch.uint8, device=DEV)
    ws.fill_(0xff)  # contents need not be initialised
    a = hc.conv_fwd_long(q, k, v, h, gs, workspace=ws).clone()
    b = hc.conv_fwd_long(q, k, v, h, gs, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_long_filter_at_width_4096_sampled_groups():
    """B=1, L=8192, D=4096, group_size 16, l_h = L (an LI-length filter):
    the whole output is computed; three groups are checked against the oracle."""
    w = WORKLOADS["se"].with_(l_h=8192, filt="se")
    log("long full: generate")
    q, k, v, h = make_inputs(w, DEV)
    y = run_long(q, k, v, h, w.group_size)
    gs = w.group_size
    for g in (0, 101, w.G - 1):
        log("  group %d" % g)
        c = slice(g * gs, (g + 1) * gs)
        sl = lambda a: a[:, :, c].contiguous().cpu()
        check_long(sl(y), sl(q), sl(k), sl(v), h[g:g + 1].cpu(), gs, w.torch_dtype, "group %d" % g)


def test_rejects_odd_width():
    q = torch.zeros(1, 16, 6, device=DEV, dtype=torch.bfloat16)
    h = torch.zeros(3, 20, device=DEV, dtype=torch.bfloat16)
    y = hc.conv_fwd_long(q, q, q, h, 2)  # D = 6 is fine
    assert torch.all(y == 0)
    q5 = torch.zeros(1, 16, 5, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(hc.HyenaError) as ei:
        hc.conv_fwd_long(q5, q5, q5, torch.zeros(5, 20, device=DEV, dtype=torch.bfloat16), 1)
    assert ei.value.status == -7


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("L,D,gs,l_h", [(1000, 64, 16, 1000), (3000, 48, 3, 700), (300, 8, 1, 5000)])
def test_kept_filter_spectra_give_the_same_bits(dt, L, D, gs, l_h):
    """hyena_conv_fwd_long_ex with reuse_spectra: a call on other inputs (and
    another batch size) with the spectra an earlier call left in the
    workspace equals a call that computes them, bit for bit; the rest of the
    workspace is filled with NaN in between."""
    dtype = DTYPES[dt]
    log("kept spectra %s L=%d D=%d gs=%d l_h=%d" % (dt, L, D, gs, l_h))
    qa, ka, va, h = (t.to(DEV) for t in gaussian_inputs(1, L, D, gs, l_h, dtype, seed=L + 1))
    qb, kb, vb, _ = (t.to(DEV) for t in gaussian_inputs(3, L, D, gs, l_h, dtype, seed=L + 2))
    code = hc.DTYPE_BF16 if dtype == torch.bfloat16 else hc.DTYPE_F32
    ws = torch.empty(hc.long_workspace_bytes(3, L, D, gs, l_h, code), dtype=torch.uint8, device=DEV)
    hc.conv_fwd_long(qa, ka, va, h, gs, workspace=ws)
    n = 1 << max(2, (L + min(l_h, L) - 2).bit_length())
    G = D // gs
    spectra = 8 * n * (G + (G & 1))
    ws[spectra:].view(torch.float32).fill_(float("nan"))
    kept = hc.conv_fwd_long(qb, kb, vb, h, gs, workspace=ws, reuse_spectra=True)
    fresh = hc.conv_fwd_long(qb, kb, vb, h, gs)
    torch.cuda.synchronize()
    assert torch.equal(kept, fresh)
    check_long(kept, qb.cpu(), kb.cpu(), vb.cpu(), h.cpu(), gs, dtype, "kept spectra")
