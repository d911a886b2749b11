"""Pins of the channel-concatenation backward oracle (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import cat_oracle as ca
from oracle import conv_oracle as co


def _flat_parts(rng, n_outer, chunks):
    return [rng.standard_normal(n_outer * c) for c in chunks]


@pytest.mark.parametrize("n_outer,chunks", [(1, [5]), (3, [4, 7]), (2, [1, 1, 9, 3]), (4, [16, 0, 8])])
def test_round_trip_against_numpy_concatenate(n_outer, chunks):
    """numpy.concatenate along the channel axis is the forward; the backward
    of every part returns that part exactly."""
    rng = np.random.default_rng(11)
    parts = _flat_parts(rng, n_outer, chunks)
    cat = np.concatenate([p.reshape(n_outer, -1) for p in parts], axis=1).reshape(-1)
    assert np.array_equal(ca.channel_cat_forward(parts, n_outer), cat)
    total, off = sum(chunks), 0
    for p, c in zip(parts, chunks):
        assert np.array_equal(ca.channel_cat_backward(cat, n_outer, c, total, off), p)
        off += c


def test_channel_slices_of_4d_tensor():
    """Inputs [B, C_k, H, W] concatenated along channels: the backward with
    chunk = C_k*H*W and offset = C_before*H*W is the channel slice."""
    rng = np.random.default_rng(12)
    B, H, W, C = 3, 4, 5, (2, 6, 3)
    dy = rng.standard_normal((B, sum(C), H, W))
    before = 0
    for c in C:
        got = ca.channel_cat_backward(dy.reshape(-1), B, c * H * W, sum(C) * H * W, before * H * W)
        assert np.array_equal(got.reshape(B, c, H, W), dy[:, before:before + c])
        before += c


def test_adjoint_and_partition():
    """<cat(x_k), dy> = sum_k <x_k, dx_k>, and the parts' gradients together
    hold every element of dy once."""
    rng = np.random.default_rng(13)
    n_outer, chunks = 5, [3, 10, 4]
    parts = _flat_parts(rng, n_outer, chunks)
    dy = rng.standard_normal(n_outer * sum(chunks))
    grads, off = [], 0
    for c in chunks:
        grads.append(ca.channel_cat_backward(dy, n_outer, c, sum(chunks), off))
        off += c
    lhs = float((ca.channel_cat_forward(parts, n_outer) * dy).sum())
    assert np.isclose(lhs, sum(float((p * g).sum()) for p, g in zip(parts, grads)), rtol=1e-12)
    assert np.array_equal(np.sort(np.concatenate(grads)), np.sort(dy))


def test_bad_ranges_raise():
    dy = np.zeros(2 * 10)
    with pytest.raises(ValueError):
        ca.channel_cat_backward(dy, 2, 4, 10, 7)
    with pytest.raises(ValueError):
        ca.channel_cat_backward(dy, 2, 4, 10, -1)


def test_conv_cat_backward_against_torch_autograd():
    """y = conv1x1(cat(x_0, x_1, x_2)) in float64 torch autograd gives the
    same part gradients and dw."""
    rng = np.random.default_rng(14)
    B, N, cout, parts_c = 2, 7, 5, [3, 1, 4]
    xs = [rng.standard_normal((B, c, N)) for c in parts_c]
    w = rng.standard_normal((cout, sum(parts_c)))
    dy = rng.standard_normal((B, cout, N))
    got, dw = ca.conv1x1_cat_backward(np.concatenate(xs, axis=1), w, dy, parts_c)
    tx = [torch.tensor(a, requires_grad=True) for a in xs]
    tw = torch.tensor(w, requires_grad=True)
    y = torch.nn.functional.conv2d(torch.cat(tx, dim=1)[..., None], tw[:, :, None, None])[..., 0]
    (y * torch.tensor(dy)).sum().backward()
    for g, t in zip(got, tx):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_conv_cat_single_part_is_conv():
    rng = np.random.default_rng(15)
    x, w, dy = rng.standard_normal((2, 6, 9)), rng.standard_normal((4, 6)), rng.standard_normal((2, 4, 9))
    (dx,), dw = ca.conv1x1_cat_backward(x, w, dy, [6])
    rx, rw = co.conv1x1_backward(x, w, dy)
    assert np.array_equal(dx, rx) and np.array_equal(dw, rw)


def test_psa_merge_round_trip_and_layout():
    """Merged channels per head: lo then hi (numpy concatenate on the
    channel axis of [B, H, half, N]); the backward returns the halves."""
    rng = np.random.default_rng(16)
    lo, hi = rng.standard_normal((2, 3, 4, 7)), rng.standard_normal((2, 3, 4, 7))
    m = ca.psa_merge_forward(lo, hi)
    assert np.array_equal(m, np.concatenate([lo, hi], axis=2))
    dlo, dhi = ca.psa_merge_backward(m)
    assert np.array_equal(dlo, lo) and np.array_equal(dhi, hi)
    # viewed as [B, H*2*half, N] (the feature map), head h's hi half starts at channel h*8 + 4
    assert np.array_equal(m.reshape(2, 24, 7)[:, 1 * 8 + 4:1 * 8 + 8], hi[:, 1])


def test_psa_merge_adjoint():
    rng = np.random.default_rng(17)
    lo, hi, dm = (rng.standard_normal((1, 2, 3, 5)), rng.standard_normal((1, 2, 3, 5)),
                  rng.standard_normal((1, 2, 6, 5)))
    dlo, dhi = ca.psa_merge_backward(dm)
    lhs = float((ca.psa_merge_forward(lo, hi) * dm).sum())
    assert np.isclose(lhs, float((lo * dlo).sum() + (hi * dhi).sum()), rtol=1e-12)
