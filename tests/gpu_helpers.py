"""Shared helpers for the GPU tests: move seeded inputs to the device, run
the HIP path through the C ABI, and compare against the oracle."""
from __future__ import annotations

import numpy as np

from oracle import psa_oracle as orc
from vision_transformer_attention_psa_amd import binding, inputs

# fp32 and bf16 bars as fixed for the method; fp16 (3 more mantissa bits
# than bf16 in the stored inputs and in the P / dS operands) gets the bf16 bar
# divided by 4.
TOL = {inputs.F32: 1e-4, inputs.BF16: 2e-2, inputs.F16: 5e-3}


def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need an MI355X"
    return t


def to_device(x: np.ndarray, bits: np.ndarray | None, dtype: str):
    t = torch()
    if dtype == inputs.BF16:
        return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).cuda()
    if dtype == inputs.F16:
        return t.from_numpy(np.ascontiguousarray(bits).view(np.float16)).cuda()
    return t.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_host(t_) -> np.ndarray:
    return t_.float().cpu().numpy().astype(np.float64)


def round_like(x: np.ndarray, dtype: str) -> np.ndarray:
    """The values a float64 array takes once stored in `dtype`."""
    f = np.asarray(x, dtype=np.float32)
    if dtype == inputs.BF16:
        return inputs.bf16_bits_to_f32(inputs.bf16_bits_rne(f)).astype(np.float64)
    if dtype == inputs.F16:
        return inputs.f16_bits_to_f32(inputs.f16_bits_rne(f)).astype(np.float64)
    return f.astype(np.float64)


def stored(x: np.ndarray, dtype: str):
    """(the float64 values of x once stored in `dtype`, a device tensor
    holding exactly those values)."""
    f = np.asarray(x, dtype=np.float32)
    if dtype == inputs.BF16:
        bits = inputs.bf16_bits_rne(f)
        return inputs.bf16_bits_to_f32(bits).astype(np.float64), to_device(None, bits, dtype)
    if dtype == inputs.F16:
        bits = inputs.f16_bits_rne(f)
        return inputs.f16_bits_to_f32(bits).astype(np.float64), to_device(None, bits, dtype)
    return f.astype(np.float64), to_device(f, None, dtype)


def device_inputs(x: inputs.Inputs):
    return to_device(x.qkv, x.qkv_bits, x.wl.dtype), to_device(x.dO, x.dO_bits, x.wl.dtype)


def run_chained(x: inputs.Inputs):
    wl = x.wl
    qkv, dO = device_inputs(x)
    o, lse = binding.fwd(qkv, wl.dk, wl.dv, wl.scale)
    d = binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale)
    torch().cuda.synchronize()
    return to_host(o), to_host(lse), to_host(d)


def errors(wl, got, ref, slices=None):
    """Per-tensor max relative errors over the chosen slices."""
    o, lse, d = got
    ro, rl, rd = ref
    dk, dv = wl.dk, wl.dv

    def pick(a):
        a = a.reshape((wl.BH,) + a.shape[2:])
        return a if slices is None else a[list(slices)]

    return {
        "O": orc.max_rel_err(pick(o), pick(ro)),
        "LSE": orc.max_rel_err(pick(lse), pick(rl)),
        "dQ": orc.max_rel_err(pick(d)[:, :dk], pick(rd)[:, :dk]),
        "dK": orc.max_rel_err(pick(d)[:, dk:2 * dk], pick(rd)[:, dk:2 * dk]),
        "dV": orc.max_rel_err(pick(d)[:, 2 * dk:], pick(rd)[:, 2 * dk:2 * dk + dv]),
    }
