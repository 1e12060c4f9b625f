"""Pins for the fp64 backward oracle (oracle.conv_bwd_ref).

Sources of truth, none of which calls the backward oracle's formulas:
  * central finite differences of the forward oracle.  The loss sum(y * dy)
    is linear in each of q, k, v and h taken alone, so the central difference
    is exact up to rounding, whatever the step.  This pins every gradient
    entry that is sampled to the forward definition;
  * torch.autograd (fp64, CPU) over a forward written with torch's grouped
    conv1d: a different implementation of the same operator;
  * closed forms: a single input impulse and a single output impulse give
    dh[s] = [s == t1 - t0], and dx is the filter read backwards.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import conv_bwd_ref, conv_fwd_ref


def _rand(rng, shape):
    return rng.standard_normal(shape)


def _loss(q, k, v, h, dy, gs):
    return float(np.sum(conv_fwd_ref(q, k, v, h, gs) * dy))


@pytest.mark.parametrize("B,L,D,gs,l_h,seed", [(1, 9, 4, 2, 3, 0), (2, 20, 6, 3, 7, 1),
                                              (1, 70, 4, 4, 66, 2)])
def test_gradients_match_central_differences_of_the_forward(B, L, D, gs, l_h, seed):
    rng = np.random.default_rng(seed)
    q, k, v, dy = (_rand(rng, (B, L, D)) for _ in range(4))
    h = _rand(rng, (D // gs, l_h))
    dq, dk, dv, dh = conv_bwd_ref(q, k, v, h, dy, gs)
    grads = {"q": dq, "k": dk, "v": dv, "h": dh}
    args = {"q": q, "k": k, "v": v, "h": h}
    eps = 0.5
    for name in ("q", "k", "v", "h"):
        a = args[name]
        idx = [tuple(rng.integers(0, n) for n in a.shape) for _ in range(12)]
        idx += [tuple([0] * a.ndim), tuple(n - 1 for n in a.shape)]
        for ix in idx:
            plus, minus = a.copy(), a.copy()
            plus[ix] += eps
            minus[ix] -= eps
            kw = dict(args)
            kw[name] = plus
            lp = _loss(kw["q"], kw["k"], kw["v"], kw["h"], dy, gs)
            kw[name] = minus
            lm = _loss(kw["q"], kw["k"], kw["v"], kw["h"], dy, gs)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grads[name][ix]) <= 1e-10 * max(1.0, abs(fd)), (name, ix)


def _torch_forward(q, k, v, h, gs):
    """y = q * (h * (k v)) with torch's grouped conv1d (cross-correlation: flip taps, pad left)."""
    B, L, D = q.shape
    G, l_h = h.shape
    w = torch.repeat_interleave(h, gs, dim=0).flip(-1)[:, None, :]  # [D, 1, l_h]
    x = (k * v).transpose(1, 2)  # [B, D, L]
    z = F.conv1d(F.pad(x, (l_h - 1, 0)), w, groups=D)
    return q * z.transpose(1, 2)


@pytest.mark.parametrize("B,L,D,gs,l_h,seed", [(2, 50, 8, 4, 7, 3), (1, 300, 16, 16, 128, 4),
                                              (3, 129, 6, 2, 65, 5)])
def test_gradients_match_torch_autograd_of_a_conv1d_forward(B, L, D, gs, l_h, seed):
    rng = np.random.default_rng(seed)
    q, k, v, dy = (_rand(rng, (B, L, D)) for _ in range(4))
    h = _rand(rng, (D // gs, l_h))
    tq, tk, tv, th = (torch.tensor(a, requires_grad=True) for a in (q, k, v, h))
    y = _torch_forward(tq, tk, tv, th, gs)
    np.testing.assert_allclose(y.detach().numpy(), conv_fwd_ref(q, k, v, h, gs), rtol=1e-11, atol=1e-11)
    y.backward(torch.tensor(dy))
    dq, dk, dv, dh = conv_bwd_ref(q, k, v, h, dy, gs)
    for got, t in ((dq, tq), (dk, tk), (dv, tv), (dh, th)):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("l_h,t0,t1", [(7, 3, 5), (128, 0, 127), (128, 64, 200), (65, 10, 10)])
def test_impulse_pair_gives_filter_gradient_at_their_distance(l_h, t0, t1):
    L, D, gs = 256, 4, 4
    k = np.ones((1, L, D))
    v = np.zeros((1, L, D))
    v[0, t0, :] = 1.0
    dy = np.zeros((1, L, D))
    dy[0, t1, :] = 1.0
    q = np.ones((1, L, D))
    h = np.random.default_rng(l_h).standard_normal((1, l_h))
    dq, dk, dv, dh = conv_bwd_ref(q, k, v, h, dy, gs)
    expect = np.zeros(l_h)
    if 0 <= t1 - t0 < l_h:
        expect[t1 - t0] = D  # four channels of the group, each contributing 1
    assert np.array_equal(dh[0], expect)
    # dx[j] = h[t1 - j] for 0 <= t1 - j < l_h; dv = dx * k with k = 1
    dx = np.zeros(L)
    for j in range(L):
        if 0 <= t1 - j < l_h:
            dx[j] = h[0, t1 - j]
    for d in range(D):
        assert np.array_equal(dv[0, :, d], dx)
        assert np.array_equal(dk[0, :, d], dx * v[0, :, d])
    # dq = dy * z: z at t1 is h[t1 - t0]
    expect_dq = np.zeros((L, D))
    if 0 <= t1 - t0 < l_h:
        expect_dq[t1] = h[0, t1 - t0]
    assert np.array_equal(dq[0], expect_dq)


def test_input_gradient_is_the_time_reversed_convolution():
    """dx of the causal conv is the same filter applied to the time-reversed dz."""
    rng = np.random.default_rng(9)
    B, L, D, gs, l_h = 2, 200, 8, 4, 100
    q, k, dy = (_rand(rng, (B, L, D)) for _ in range(3))
    v = np.ones((B, L, D))
    h = _rand(rng, (D // gs, l_h))
    _, dk, _, _ = conv_bwd_ref(q, k, v, h, dy, gs)  # dk = dx * v = dx
    rev = lambda a: a[:, ::-1, :]
    ones = np.ones((B, L, D))
    dx_rev = conv_fwd_ref(ones, rev(dy), rev(q), h, gs)  # causal conv of reversed dz = dy*q
    np.testing.assert_allclose(dk, rev(dx_rev), rtol=1e-12, atol=1e-12)


def test_empty_and_degenerate():
    a = np.zeros((1, 0, 4))
    dq, dk, dv, dh = conv_bwd_ref(a, a, a, np.ones((2, 3)), a, 2)
    assert dq.shape == (1, 0, 4) and np.all(dh == 0)
    rng = np.random.default_rng(1)
    q, k, v, dy = (_rand(rng, (1, 5, 2)) for _ in range(4))
    h = _rand(rng, (1, 1))  # one tap: y = h0 q k v
    dq, dk, dv, dh = conv_bwd_ref(q, k, v, h, dy, 2)
    np.testing.assert_allclose(dq, dy * h[0, 0] * k * v, rtol=1e-15)
    np.testing.assert_allclose(dk, dy * q * h[0, 0] * v, rtol=1e-15)
    np.testing.assert_allclose(dh[0, 0], np.sum(dy * q * k * v), rtol=1e-13)
