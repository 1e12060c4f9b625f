"""Pins for the fp64 oracle: each test ties it to something other than itself.

Sources of truth used here (none of them calls the oracle's own formula):
  * the worked example printed on the page "04. hardware-aware convolution
    kernels", section 3 (tests/golden/worked_example.txt);
  * numpy.convolve (textbook linear convolution), numpy.fft (convolution
    theorem) and scipy.linalg.toeplitz (the Toeplitz form of section 1);
  * closed forms and invariants: impulse response, constant input, linearity,
    causality, shift equivariance, batch isolation, group sharing, gating order.

The set is chosen so that the plausible mistakes fail at least one test: a
dropped or extra tap (impulse, constant input, convolve), a flipped filter
(impulse, worked example), q applied before instead of after the convolution
(gating order), a wrong filter-to-channel map (group map), history leaking
across batch rows (batch isolation) or from the future (causality).
"""
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import conv_fwd_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.txt")


def _load_worked_example():
    meta, mats, cur = {}, {}, None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] in ("l", "l_h", "l_b"):
                meta[parts[0]] = int(parts[1])
            elif parts[0] in ("H0", "H1"):
                cur = parts[0]
                mats[cur] = []
            else:
                mats[cur].append(parts)
    return meta, mats


def _symbolic(rows, taps):
    out = np.zeros((len(rows), len(rows[0])))
    for i, row in enumerate(rows):
        for j, s in enumerate(row):
            out[i, j] = 0.0 if s == "0" else taps[int(s[1:])]
    return out


def _toeplitz_from_impulses(taps, L):
    """Column j of the operator's matrix = its output for an impulse at j (q = k = 1)."""
    T = np.zeros((L, L))
    for j in range(L):
        v = np.zeros((1, L, 1))
        v[0, j, 0] = 1.0
        ones = np.ones_like(v)
        T[:, j] = conv_fwd_ref(ones, ones, v, np.asarray(taps)[None, :], 1)[0, :, 0]
    return T


# --------------------------------------------------------------------------
# Worked example of section 3 (l = 6, l_h = 4, l_b = 3)
# --------------------------------------------------------------------------

def test_worked_example_blocks_match_printed_H0_H1():
    meta, mats = _load_worked_example()
    L, l_h, l_b = meta["l"], meta["l_h"], meta["l_b"]
    assert (L, l_h, l_b) == (6, 4, 3)
    taps = np.array([3.0, 5.0, 7.0, 11.0])  # distinct, so every entry names its tap
    T = _toeplitz_from_impulses(taps, L)
    H0 = _symbolic(mats["H0"], taps)
    H1 = _symbolic(mats["H1"], taps)
    assert np.array_equal(T[0:l_b, 0:l_b], H0)
    assert np.array_equal(T[l_b:2 * l_b, l_b:2 * l_b], H0)
    assert np.array_equal(T[l_b:2 * l_b, 0:l_b], H1)
    assert np.all(T[0:l_b, l_b:2 * l_b] == 0.0)  # causal: nothing above the diagonal


def test_worked_example_two_stage_reproduces_output():
    meta, mats = _load_worked_example()
    L, l_b = meta["l"], meta["l_b"]
    rng = np.random.default_rng(7)
    taps = rng.standard_normal(meta["l_h"])
    H0 = _symbolic(mats["H0"], taps)
    H1 = _symbolic(mats["H1"], taps)
    x = rng.standard_normal(L)
    ones = np.ones((1, L, 1))
    y = conv_fwd_ref(ones, ones, x[None, :, None], taps[None, :], 1)[0, :, 0]
    X0, X1 = x[:l_b], x[l_b:]
    np.testing.assert_allclose(y[:l_b], H0 @ X0, rtol=0, atol=1e-14)  # no block before chunk 0
    np.testing.assert_allclose(y[l_b:], H0 @ X1 + H1 @ X0, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# Library routines
# --------------------------------------------------------------------------

@pytest.mark.parametrize("L,D,gs,l_h,seed", [
    (1, 3, 1, 1, 0), (6, 2, 2, 4, 1), (100, 8, 4, 7, 2), (257, 6, 3, 128, 3),
    (300, 16, 16, 65, 4), (64, 4, 1, 64, 5), (65, 2, 1, 66, 6),
    # long filters (the FFT path's regime): as long as the sequence, and longer
    (300, 4, 2, 300, 7), (200, 2, 1, 500, 8)])
def test_matches_numpy_convolve_exactly_on_integers(L, D, gs, l_h, seed):
    rng = np.random.default_rng(seed)
    v = rng.integers(-3, 4, size=(1, L, D)).astype(np.float64)
    h = rng.integers(-3, 4, size=(D // gs, l_h)).astype(np.float64)
    ones = np.ones_like(v)
    y = conv_fwd_ref(ones, ones, v, h, gs)
    for d in range(D):
        ref = np.convolve(v[0, :, d], h[d // gs])[:L]
        assert np.array_equal(y[0, :, d], ref)


@pytest.mark.parametrize("B,L,D,gs,l_h,seed", [
    (1, 512, 16, 16, 7, 10), (2, 333, 32, 16, 128, 11), (3, 129, 8, 2, 100, 12),
    (1, 1000, 4, 1, 1000, 13), (2, 700, 6, 3, 1500, 14)])
def test_matches_fft_convolution(B, L, D, gs, l_h, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, L, D)) for _ in range(3))
    h = rng.standard_normal((D // gs, l_h))
    y = conv_fwd_ref(q, k, v, h, gs)
    n = 1 << int(np.ceil(np.log2(L + l_h - 1)))
    x = k * v
    hx = np.repeat(h, gs, axis=0)  # [D, l_h]
    X = np.fft.rfft(x, n=n, axis=1)
    H = np.fft.rfft(hx.T, n=n, axis=0)[None]
    z = np.fft.irfft(X * H, n=n, axis=1)[:, :L, :]
    ref = q * z
    assert np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("L,l_h,seed", [(40, 7, 20), (200, 128, 21), (130, 65, 22)])
def test_matches_dense_toeplitz_matrix(L, l_h, seed):
    rng = np.random.default_rng(seed)
    D, gs = 4, 2
    q, k, v = (rng.standard_normal((1, L, D)) for _ in range(3))
    h = rng.standard_normal((D // gs, l_h))
    y = conv_fwd_ref(q, k, v, h, gs)
    for d in range(D):
        col = np.zeros(L)
        col[:min(L, l_h)] = h[d // gs][:min(L, l_h)]
        T = scipy.linalg.toeplitz(col, np.zeros(L))  # lower-triangular Toeplitz
        ref = q[0, :, d] * (T @ (k[0, :, d] * v[0, :, d]))
        np.testing.assert_allclose(y[0, :, d], ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Closed forms and invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("l_h", [1, 7, 64, 65, 127, 128])
def test_impulse_gives_filter_at_chunk_seams(l_h):
    L = 300
    rng = np.random.default_rng(l_h)
    h = rng.standard_normal((1, l_h))
    for t0 in (0, 63, 64, 127, 128, L - 1):
        v = np.zeros((1, L, 1))
        v[0, t0, 0] = 1.0
        ones = np.ones_like(v)
        z = conv_fwd_ref(ones, ones, v, h, 1)[0, :, 0]
        expect = np.zeros(L)
        n = min(l_h, L - t0)
        expect[t0:t0 + n] = h[0, :n]
        assert np.array_equal(z, expect)


def test_last_tap_only_filter_reaches_back_l_h_minus_1():
    L, l_h = 400, 128
    h = np.zeros((1, l_h))
    h[0, l_h - 1] = 1.0
    rng = np.random.default_rng(3)
    v = rng.standard_normal((1, L, 1))
    ones = np.ones_like(v)
    z = conv_fwd_ref(ones, ones, v, h, 1)[0, :, 0]
    assert np.array_equal(z[:l_h - 1], np.zeros(l_h - 1))
    assert np.array_equal(z[l_h - 1:], v[0, :L - l_h + 1, 0])


@pytest.mark.parametrize("l_h", [1, 7, 128])
def test_constant_input_gives_partial_sums_of_filter(l_h):
    L = 200
    h = np.arange(1, l_h + 1, dtype=np.float64)[None, :]
    ones = np.ones((1, L, 1))
    z = conv_fwd_ref(ones, ones, ones, h, 1)[0, :, 0]
    t = np.arange(L)
    m = np.minimum(t, l_h - 1) + 1  # number of taps seen at time t
    assert np.array_equal(z, m * (m + 1) / 2.0)  # 1 + 2 + ... + m


def test_single_tap_is_elementwise_product():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((2, 50, 6)) for _ in range(3))
    h = rng.standard_normal((3, 1))
    y = conv_fwd_ref(q, k, v, h, 2)
    hd = np.repeat(h[:, 0], 2)[None, None, :]
    np.testing.assert_allclose(y, hd * q * k * v, rtol=1e-15, atol=0)


def test_gating_applies_q_after_the_convolution():
    L, l_h = 90, 40
    rng = np.random.default_rng(5)
    h = rng.standard_normal((1, l_h))
    t0, t1 = 20, 47
    q = np.zeros((1, L, 1)); q[0, t1, 0] = 2.0
    v = np.zeros((1, L, 1)); v[0, t0, 0] = 3.0
    k = np.full((1, L, 1), 0.5)
    y = conv_fwd_ref(q, k, v, h, 1)[0, :, 0]
    expect = np.zeros(L)
    expect[t1] = 2.0 * h[0, t1 - t0] * 0.5 * 3.0
    assert np.array_equal(y, expect)


def test_linearity_in_q_x_and_h():
    rng = np.random.default_rng(6)
    B, L, D, gs, l_h = 1, 150, 8, 4, 70
    q, k, v1, v2 = (rng.standard_normal((B, L, D)) for _ in range(4))
    h1, h2 = rng.standard_normal((2, D // gs, l_h))
    a, b = 1.75, -0.5
    f = lambda qq, vv, hh: conv_fwd_ref(qq, k, vv, hh, gs)
    tol = dict(rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f(q, a * v1 + b * v2, h1), a * f(q, v1, h1) + b * f(q, v2, h1), **tol)
    np.testing.assert_allclose(f(q, v1, a * h1 + b * h2), a * f(q, v1, h1) + b * f(q, v1, h2), **tol)
    np.testing.assert_allclose(f(a * q, v1, h1), a * f(q, v1, h1), **tol)


def test_causality_and_finite_support():
    rng = np.random.default_rng(8)
    B, L, D, gs, l_h = 1, 300, 4, 4, 128
    q, k, v = (rng.standard_normal((B, L, D)) for _ in range(3))
    h = rng.standard_normal((1, l_h))
    y0 = conv_fwd_ref(q, k, v, h, gs)
    t0 = 100
    v2 = v.copy()
    v2[:, t0, :] += 5.0
    y1 = conv_fwd_ref(q, k, v2, h, gs)
    assert np.array_equal(y0[:, :t0], y1[:, :t0])
    assert np.array_equal(y0[:, t0 + l_h:], y1[:, t0 + l_h:])
    assert np.all(y0[:, t0:t0 + l_h] != y1[:, t0:t0 + l_h])


def test_first_output_uses_only_first_input():
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((2, 10, 4)) for _ in range(3))
    h = rng.standard_normal((2, 5))
    y = conv_fwd_ref(q, k, v, h, 2)
    hd = np.repeat(h[:, 0], 2)
    np.testing.assert_allclose(y[:, 0, :], q[:, 0, :] * hd * k[:, 0, :] * v[:, 0, :], rtol=1e-15)


def test_shift_equivariance():
    rng = np.random.default_rng(10)
    L, m, l_h = 200, 37, 50
    q, k, v = (rng.standard_normal((1, L, 2)) for _ in range(3))
    h = rng.standard_normal((1, l_h))
    shift = lambda a: np.concatenate([np.zeros((1, m, 2)), a[:, :L - m]], axis=1)
    y = conv_fwd_ref(q, k, v, h, 2)
    ys = conv_fwd_ref(shift(q), shift(k), shift(v), h, 2)
    np.testing.assert_allclose(ys[:, m:], y[:, :L - m], rtol=1e-13, atol=1e-13)
    assert np.all(ys[:, :m] == 0.0)


def test_batch_rows_are_isolated():
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((2, 120, 4)) for _ in range(3))
    k[1] = 0.0
    h = rng.standard_normal((1, 100))
    y = conv_fwd_ref(q, k, v, h, 4)
    assert np.all(y[1] == 0.0)
    y0 = conv_fwd_ref(q[:1], k[:1], v[:1], h, 4)
    assert np.array_equal(y[:1], y0)


def test_group_map_is_channel_floordiv_group_size():
    L, D, gs, l_h = 20, 6, 3, 4
    h = np.array([[1.0, 2.0, 3.0, 4.0], [10.0, 20.0, 30.0, 40.0]])
    for d in range(D):
        v = np.zeros((1, L, D))
        v[0, 0, d] = 1.0
        ones = np.ones_like(v)
        y = conv_fwd_ref(ones, ones, v, h, gs)
        assert np.array_equal(y[0, :l_h, d], h[d // gs])
        others = [c for c in range(D) if c != d]
        assert np.all(y[0, :, others] == 0.0)


def test_channels_sharing_a_group_give_equal_outputs():
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((1, 80, 1)) for _ in range(3))
    rep = lambda a: np.repeat(a, 4, axis=2)
    h = rng.standard_normal((1, 9))
    y = conv_fwd_ref(rep(q), rep(k), rep(v), h, 4)
    for d in range(1, 4):
        assert np.array_equal(y[..., d], y[..., 0])


def test_empty_shapes():
    for shape in [(0, 5, 4), (1, 0, 4), (1, 5, 0)]:
        a = np.zeros(shape)
        G = max(shape[2] // 2, 0)
        y = conv_fwd_ref(a, a, a, np.zeros((G, 3)), 2)
        assert y.shape == shape


def test_rejects_inconsistent_shapes():
    a = np.zeros((1, 4, 6))
    with pytest.raises(ValueError):
        conv_fwd_ref(a, a, a, np.zeros((2, 3)), 4)  # 6 % 4 != 0
    with pytest.raises(ValueError):
        conv_fwd_ref(a, a, a, np.zeros((2, 3)), 2)  # 3 filters needed
