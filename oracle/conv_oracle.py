"""CPU oracle for the backward of the 1x1 convolution that produces the
packed attention projection (float64).

TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark may import
this module.  It shares no code with the HIP path.

Source: the Conv2dBackward page (teenygrad conv2d kernels), struct
description: one pass computes both input and weight gradients of a 2-D
convolution, dx accumulating dy * w and dw accumulating the sum of dy * x.
The attention block's projection is that convolution with a 1 x 1 kernel,
stride 1, no padding and one group (g = 1), so per batch b and token n

    y[b][co][n]  = sum_ci w[co][ci] x[b][ci][n]
    dx[b][ci][n] = sum_co w[co][ci] dy[b][co][n]
    dw[co][ci]   = sum_b sum_n dy[b][co][n] x[b][ci][n]

Each is written as its definition with whole-matrix numpy products; the
page's atomics (which need zeroed outputs) have no counterpart here.
"""
from __future__ import annotations

import numpy as np


def conv1x1_forward(x, w):
    """y [B, cout, N] from x [B, cin, N] and w [cout, cin]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return np.einsum("oc,bcn->bon", w, x)


def conv1x1_backward(x, w, dy):
    """(dx [B, cin, N], dw [cout, cin]) for upstream gradient dy [B, cout, N]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64).reshape(x.shape[0], w.shape[0], x.shape[2])
    dx = np.stack([w.T @ dy[b] for b in range(x.shape[0])])
    dw = sum(dy[b] @ x[b].T for b in range(x.shape[0]))
    return dx, dw
