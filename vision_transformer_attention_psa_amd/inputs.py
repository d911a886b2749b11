"""Seeded synthetic workloads for PSA self-attention over a conv feature map.

This module only draws and rounds random numbers; it holds none of the
attention arithmetic, so the CPU oracle and the HIP path can both be fed from
it without sharing any of the method's code.

Layout (PsaFa2Backward page, struct description: one (n, bh) pair per work
item, N_CTX_Q == N_CTX_K == N): the packed projection ``qkv`` is channel-major,
``[B, heads, 2*dk + dv, N]`` with the N = H*W tokens contiguous; channels
``[0, dk)`` are Q, ``[dk, 2*dk)`` are K and ``[2*dk, 2*dk + dv)`` are V.  The
upstream gradient ``dO`` is ``[B, heads, dv, N]`` in the same orientation.

Recipe: ``numpy.random.Generator(PCG64(seed))`` draws ``qkv`` then ``dO`` as
float32 standard normals; the high-resolution workload scales the Q and K
channels by 3.  bf16 and fp16 workloads round both tensors to the storage
type with round-to-nearest-even, and those exact values are what every
consumer sees.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"
F16 = "f16"
HALF = (BF16, F16)  # 16-bit storage types


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    H: int
    W: int
    dk: int
    dv: int
    dtype: str
    seed: int
    sigma_qk: float = 1.0

    @property
    def N(self) -> int:
        return self.H * self.W

    @property
    def BH(self) -> int:
        return self.B * self.heads

    @property
    def channels(self) -> int:
        return 2 * self.dk + self.dv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dk)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five feature-map shapes a YOLO PSA block sees (8x8 up to 80x80 maps).
WORKLOADS = {
    "tiny_n64_f32": Workload("tiny_n64_f32", B=1, heads=1, H=8, W=8, dk=16, dv=16,
                             dtype=F32, seed=1),
    "nano_n400_f32": Workload("nano_n400_f32", B=1, heads=2, H=20, W=20, dk=32, dv=64,
                              dtype=F32, seed=2),
    "batched_n400_bf16": Workload("batched_n400_bf16", B=16, heads=4, H=20, W=20, dk=32,
                                  dv=64, dtype=BF16, seed=3),
    "midres_n1600_bf16": Workload("midres_n1600_bf16", B=8, heads=8, H=40, W=40, dk=32,
                                  dv=64, dtype=BF16, seed=4),
    "highres_n6400_bf16": Workload("highres_n6400_bf16", B=4, heads=8, H=80, W=80, dk=64,
                                   dv=64, dtype=BF16, seed=5, sigma_qk=3.0),
}
WORKLOAD_ORDER = list(WORKLOADS)


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN inputs map to a quiet NaN; finite values that round past the largest
    bf16 become +-inf, as IEEE rounding prescribes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f16_bits_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (uint16), round to nearest even
    (numpy's float16 conversion), overflow to +-inf."""
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of binary16 bit patterns to float32."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


@dataclasses.dataclass
class Inputs:
    """One draw of a workload.

    ``qkv``/``dO`` are float32 arrays holding exactly the values the kernels
    see (already representable in the storage type for 16-bit workloads);
    ``qkv_bits`` and ``dO_bits`` hold the uint16 patterns for bf16 and fp16
    workloads, else ``None``.
    """

    wl: Workload
    qkv: np.ndarray
    dO: np.ndarray
    qkv_bits: np.ndarray | None
    dO_bits: np.ndarray | None


def make_inputs(wl: Workload, seed: int | None = None) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    qkv = rng.standard_normal((wl.B, wl.heads, wl.channels, wl.N), dtype=np.float32)
    dO = rng.standard_normal((wl.B, wl.heads, wl.dv, wl.N), dtype=np.float32)
    if wl.sigma_qk != 1.0:
        qkv[:, :, : 2 * wl.dk, :] *= np.float32(wl.sigma_qk)
    if wl.dtype == BF16:
        qb, db = bf16_bits_rne(qkv), bf16_bits_rne(dO)
        return Inputs(wl, bf16_bits_to_f32(qb), bf16_bits_to_f32(db), qb, db)
    if wl.dtype == F16:
        qb, db = f16_bits_rne(qkv), f16_bits_rne(dO)
        return Inputs(wl, f16_bits_to_f32(qb), f16_bits_to_f32(db), qb, db)
    return Inputs(wl, qkv, dO, None, None)


def sample_slices(wl: Workload, count: int, seed: int = 0) -> list[int]:
    """A fixed, seeded choice of (b*heads + h) slice indices, always including
    the first and the last slice so both ends of the batch are covered."""
    if count >= wl.BH:
        return list(range(wl.BH))
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    mid = rng.choice(np.arange(1, wl.BH - 1), size=max(0, count - 2), replace=False)
    return sorted({0, wl.BH - 1, *map(int, mid)})


@dataclasses.dataclass
class ConvInputs:
    """One draw for the 1x1-convolution backward: x [B, cin, N], w [cout, cin]
    and dy [B, cout, N] as float32 values exactly representable in `dtype`,
    with the uint16 patterns for 16-bit dtypes (else None)."""

    dtype: str
    x: np.ndarray
    w: np.ndarray
    dy: np.ndarray
    bits: tuple | None


def make_conv_inputs(B: int, cin: int, cout: int, N: int, dtype: str, seed: int) -> ConvInputs:
    """Standard normals for x and dy and N(0, 1/cin) weights (the usual
    fan-in scaling), drawn x, w, dy in that order, then rounded like the
    attention inputs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, cin, N), dtype=np.float32)
    w = rng.standard_normal((cout, cin), dtype=np.float32) * np.float32(1.0 / math.sqrt(cin))
    dy = rng.standard_normal((B, cout, N), dtype=np.float32)
    if dtype == BF16:
        bits = tuple(bf16_bits_rne(a) for a in (x, w, dy))
        return ConvInputs(dtype, *(bf16_bits_to_f32(b) for b in bits), bits)
    if dtype == F16:
        bits = tuple(f16_bits_rne(a) for a in (x, w, dy))
        return ConvInputs(dtype, *(f16_bits_to_f32(b) for b in bits), bits)
    return ConvInputs(dtype, x, w, dy, None)
