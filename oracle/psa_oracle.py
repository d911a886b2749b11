"""CPU oracle for PSA self-attention forward and backward (float64).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module.  It shares no code
with the HIP path and must never be reached from the product path.

What it computes, and from where:

* PsaFa2Backward page (vision_rs psa kernels), struct description: a combined
  Flash-Attention-2 backward for self-attention in which the query and key
  sequences are the same N tokens (N_CTX_Q == N_CTX_K == N) and every query
  visits every key row, so attention is full and non-causal.  The page names
  the method (FlashAttention-2) but prints no formula; the plainest reading is
  the standard softmax attention it computes exactly:

      S = s * Q K^T                     (N x N, s = softmax scale)
      LSE_i = log sum_j exp(S_ij)       (natural log, scale included)
      P = exp(S - LSE)                  (rows sum to 1, softmax over keys)
      O = P V

  and its exact gradient for an upstream gradient dO:

      D_i  = sum_c dO_ic O_ic
      dP   = dO V^T
      dS   = P o (dP - D)
      dQ   = s dS K,   dK = s dS^T Q,   dV = P^T dO.

* The same description fixes the output buffer: one packed gradient with
  section 0 = dQ, section 1 = dK, section 2 = dV, laid out exactly like the
  packed input, [B, heads, 2*dk + dv, N], channel-major (token contiguous).
  The page accumulates sections 0 and 1 from two calls (a lo and a hi half
  of V); the sum of those two calls is the single-call gradient written here.

Each step is written as its definition with whole-matrix numpy operations on
one (batch, head) slice at a time; nothing is blocked, fused or reordered.
"""
from __future__ import annotations

import numpy as np


def _slice_views(qkv_bh: np.ndarray, dk: int, dv: int):
    """Split one channel-major packed slice [2dk+dv, N] into token-major
    Q [N, dk], K [N, dk], V [N, dv] (float64)."""
    x = np.asarray(qkv_bh, dtype=np.float64)
    assert x.shape[0] == 2 * dk + dv
    return x[:dk].T, x[dk:2 * dk].T, x[2 * dk:2 * dk + dv].T


def forward_slice(qkv_bh, dk: int, dv: int, scale: float):
    """One (batch, head) slice.  Returns O [dv, N] and LSE [N] (float64)."""
    Q, K, V = _slice_views(qkv_bh, dk, dv)
    S = scale * (Q @ K.T)
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    P = np.exp(S - lse[:, None])
    O = P @ V
    return O.T.copy(), lse


def backward_slice(qkv_bh, o_bh, lse_bh, dO_bh, dk: int, dv: int, scale: float):
    """One (batch, head) slice of the backward, recomputing P from LSE.

    ``o_bh`` [dv, N] is the forward output as given (D is formed from it),
    ``lse_bh`` [N] the natural-log row logsumexp, ``dO_bh`` [dv, N].
    Returns the packed gradient slice [2*dk + dv, N] (float64).
    """
    Q, K, V = _slice_views(qkv_bh, dk, dv)
    O = np.asarray(o_bh, dtype=np.float64).T
    G = np.asarray(dO_bh, dtype=np.float64).T
    lse = np.asarray(lse_bh, dtype=np.float64)
    P = np.exp(scale * (Q @ K.T) - lse[:, None])
    D = (G * O).sum(axis=1)
    dP = G @ V.T
    dS = P * (dP - D[:, None])
    dQ = scale * (dS @ K)
    dK = scale * (dS.T @ Q)
    dV = P.T @ G
    return np.concatenate([dQ.T, dK.T, dV.T], axis=0)


def _pick(n_slices: int, slices):
    return range(n_slices) if slices is None else list(slices)


def forward(qkv, dk: int, dv: int, scale: float, slices=None):
    """Packed forward.  ``qkv`` [B, heads, 2dk+dv, N].

    Returns ``o`` [B, heads, dv, N] and ``lse`` [B, heads, N] in float64.
    With ``slices`` (flat b*heads + h indices) only those slices are
    computed; the others are left as NaN.
    """
    qkv = np.asarray(qkv)
    B, H, C, N = qkv.shape
    assert C == 2 * dk + dv
    flat = qkv.reshape(B * H, C, N)
    o = np.full((B * H, dv, N), np.nan)
    lse = np.full((B * H, N), np.nan)
    for s in _pick(B * H, slices):
        o[s], lse[s] = forward_slice(flat[s], dk, dv, scale)
    return o.reshape(B, H, dv, N), lse.reshape(B, H, N)


def backward(qkv, o, lse, dO, dk: int, dv: int, scale: float, slices=None):
    """Packed backward from the forward's (o, lse).  Returns d_packed
    [B, heads, 2dk+dv, N] in float64 (NaN outside ``slices`` if given)."""
    qkv = np.asarray(qkv)
    B, H, C, N = qkv.shape
    flat = qkv.reshape(B * H, C, N)
    of = np.asarray(o).reshape(B * H, dv, N)
    lf = np.asarray(lse).reshape(B * H, N)
    gf = np.asarray(dO).reshape(B * H, dv, N)
    d = np.full((B * H, C, N), np.nan)
    for s in _pick(B * H, slices):
        d[s] = backward_slice(flat[s], of[s], lf[s], gf[s], dk, dv, scale)
    return d.reshape(B, H, C, N)


def forward_backward(qkv, dO, dk: int, dv: int, scale: float, slices=None):
    """Forward then backward on the oracle's own float64 (o, lse)."""
    o, lse = forward(qkv, dk, dv, scale, slices)
    return o, lse, backward(qkv, o, lse, dO, dk, dv, scale, slices)


def preprocess_D(o, dO):
    """D = rowsum(dO o O) per query, [B, heads, N] (float64)."""
    return (np.asarray(o, dtype=np.float64) * np.asarray(dO, dtype=np.float64)).sum(axis=2)


def max_rel_err(got, ref) -> float:
    """Per-tensor error: max |got - ref| / max |ref| over the whole tensor.

    Elementwise relative error is ill-posed here: rows of dS sum to zero, so
    dQ and dK entries cross zero.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.abs(ref).max()
    if denom == 0.0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / denom)
