"""CPU oracle for the channel-concatenation backward, alone and composed
with the 1x1-convolution backward (exact copies, float64 for the product).

TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark may import
this module.  It shares no code with the HIP path.

Source: the ChannelCatBackward page (teenygrad channel_cat kernels), struct
description.  The combined gradient dy of a concatenation holds, for every
outer index n, total contiguous elements; one input's gradient is the chunk
elements that start at offset within each of them:

    dx[n * chunk + e] = dy[n * total + offset + e],   e < chunk

The page gives that index mapping and says the forward (channel_cat_forward)
runs on the same grid, so the forward here is the same mapping read the
other way: input k's elements are placed at offset_k of every outer row.
"""
from __future__ import annotations

import numpy as np

from .conv_oracle import conv1x1_backward


def channel_cat_forward(parts, n_outer: int):
    """Flat concatenation of flat inputs: parts[k] holds n_outer * chunk_k
    elements; the result holds n_outer * sum(chunk_k), input k's row n at
    n * total + offset_k."""
    chunks = [len(p) // n_outer for p in parts]
    total = sum(chunks)
    out = np.empty(n_outer * total, dtype=np.result_type(*parts))
    offset = 0
    for p, chunk in zip(parts, chunks):
        for n in range(n_outer):
            out[n * total + offset: n * total + offset + chunk] = p[n * chunk:(n + 1) * chunk]
        offset += chunk
    return out


def channel_cat_backward(dy, n_outer: int, chunk: int, total: int, offset: int):
    """The page's index mapping: dx[n * chunk + e] = dy[n * total + offset + e]."""
    dy = np.asarray(dy).reshape(-1)
    if offset < 0 or offset + chunk > total or dy.size != n_outer * total:
        raise ValueError("need 0 <= offset, offset + chunk <= total, dy of n_outer * total elements")
    dx = np.empty(n_outer * chunk, dtype=dy.dtype)
    for n in range(n_outer):  # all e < chunk of row n at once
        dx[n * chunk:(n + 1) * chunk] = dy[n * total + offset:n * total + offset + chunk]
    return dx


def conv1x1_cat_backward(x, w, dy, part_channels):
    """Backward of y = w cat(x_0, ..., x_{K-1}) for a 1x1 convolution: the
    convolution's (dx, dw), then the concatenation's backward for each part
    (outer index = batch, chunk = c_k * N, total = cin * N, offset = c_before * N).
    Returns ([dx_0, ..., dx_{K-1}] each [B, c_k, N], dw)."""
    dx, dw = conv1x1_backward(x, w, dy)
    B, cin, N = dx.shape
    if sum(part_channels) != cin:
        raise ValueError("part channels must add up to cin")
    out, before = [], 0
    for c in part_channels:
        flat = channel_cat_backward(dx.reshape(-1), B, c * N, cin * N, before * N)
        out.append(flat.reshape(B, c, N))
        before += c
    return out, dw


def psa_merge_forward(o_lo, o_hi):
    """PsaMergeAttnRuntimeOp page (the op joining the two attention calls'
    outputs), read as a per-head channel concatenation: merged[b][h] holds
    o_lo[b][h]'s channels, then o_hi[b][h]'s.  [B, H, half, N] each ->
    [B, H, 2*half, N]."""
    B, H, half, N = np.shape(o_lo)
    flat = channel_cat_forward([np.asarray(o_lo).reshape(-1), np.asarray(o_hi).reshape(-1)], B * H)
    return flat.reshape(B, H, 2 * half, N)


def psa_merge_backward(d_merged):
    """The merge's backward: each head's channel halves of d_merged
    [B, H, 2*half, N], as (d_lo, d_hi) [B, H, half, N]."""
    B, H, C, N = np.shape(d_merged)
    half = C // 2
    flat = np.asarray(d_merged).reshape(-1)
    lo = channel_cat_backward(flat, B * H, half * N, C * N, 0)
    hi = channel_cat_backward(flat, B * H, half * N, C * N, half * N)
    return lo.reshape(B, H, half, N), hi.reshape(B, H, half, N)
