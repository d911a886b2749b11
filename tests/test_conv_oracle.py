"""Pins of the 1x1-convolution backward oracle (CPU only)."""
import numpy as np
import pytest

from oracle import conv_oracle as co


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_finite_differences():
    """L = <dy, conv(x, w)>: central differences in every element of x and w."""
    rng = np.random.default_rng(7)
    B, cin, cout, N = 2, 3, 4, 5
    x, w, dy = _rand(rng, B, cin, N), _rand(rng, cout, cin), _rand(rng, B, cout, N)
    dx, dw = co.conv1x1_backward(x, w, dy)

    def L(x_, w_):
        return float((dy * co.conv1x1_forward(x_, w_)).sum())

    h = 1e-6
    for arr, grad, is_x in ((x, dx, True), (w, dw, False)):
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            fd = (L(p, w) - L(m, w)) / (2 * h) if is_x else (L(x, p) - L(x, m)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(grad).max())


def test_adjoint_identity():
    """L is bilinear, so <dx, x> = <dw, w> = <dy, y>."""
    rng = np.random.default_rng(8)
    x, w, dy = _rand(rng, 3, 16, 33), _rand(rng, 24, 16), _rand(rng, 3, 24, 33)
    dx, dw = co.conv1x1_backward(x, w, dy)
    L = float((dy * co.conv1x1_forward(x, w)).sum())
    assert np.isclose((dx * x).sum(), L, rtol=1e-12)
    assert np.isclose((dw * w).sum(), L, rtol=1e-12)


def test_closed_form_ones():
    """x = 1, dy = 1: dw = B*N everywhere and dx[ci] = sum_co w[co][ci]."""
    rng = np.random.default_rng(9)
    B, cin, cout, N = 2, 5, 7, 11
    w = _rand(rng, cout, cin)
    dx, dw = co.conv1x1_backward(np.ones((B, cin, N)), w, np.ones((B, cout, N)))
    assert np.array_equal(dw, np.full((cout, cin), float(B * N)))
    np.testing.assert_allclose(dx, np.broadcast_to(w.sum(axis=0)[None, :, None], (B, cin, N)), rtol=1e-14)


def test_packed_gradient_view():
    """dy given as a packed gradient [B, heads, 2dk+dv, N] is read as [B, cout, N]."""
    rng = np.random.default_rng(10)
    B, heads, C, N, cin = 2, 3, 8, 6, 4
    x, w = _rand(rng, B, cin, N), _rand(rng, heads * C, cin)
    dy = _rand(rng, B, heads, C, N)
    a = co.conv1x1_backward(x, w, dy)
    b = co.conv1x1_backward(x, w, dy.reshape(B, heads * C, N))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_against_torch_conv2d_autograd():
    """Library cross-check: torch float64 conv2d with a 1x1 kernel."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    B, cin, cout, H, W = 2, 6, 10, 3, 4
    x, w, dy = _rand(rng, B, cin, H * W), _rand(rng, cout, cin), _rand(rng, B, cout, H * W)
    xt = torch.tensor(x.reshape(B, cin, H, W), requires_grad=True)
    wt = torch.tensor(w.reshape(cout, cin, 1, 1), requires_grad=True)
    y = torch.nn.functional.conv2d(xt, wt)
    y.backward(torch.tensor(dy.reshape(B, cout, H, W)))
    dx, dw = co.conv1x1_backward(x, w, dy)
    np.testing.assert_allclose(dx, xt.grad.numpy().reshape(B, cin, H * W), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy().reshape(cout, cin), rtol=1e-12, atol=1e-12)
