"""psa_attn_bwd_noalloc (statistics in the library's static device array,
no allocation) against psa_attn_bwd on the same inputs through the C ABI:
two calls in a row, the second on a smaller problem, each bitwise equal to
the allocating entry point (same kernels, same inputs) and within the
parity bar of the oracle."""
import numpy as np
import pytest

from oracle import psa_oracle as orc
from vision_transformer_attention_psa_amd import binding, inputs

from gpu_helpers import TOL, device_inputs, to_host, torch

pytestmark = pytest.mark.gpu

CODES = {inputs.F32: binding.PSA_F32, inputs.BF16: binding.PSA_BF16, inputs.F16: binding.PSA_F16}


def _noalloc(qkv, o, lse, dO, wl):
    t = torch()
    d = t.full_like(qkv, float("nan"))
    rc = binding.psa_attn_bwd_noalloc(qkv.data_ptr(), o.data_ptr(), lse.data_ptr(), dO.data_ptr(), d.data_ptr(),
                                      wl.B, wl.heads, wl.N, wl.dk, wl.dv, float(wl.scale), CODES[wl.dtype],
                                      t.cuda.current_stream().cuda_stream)
    assert rc == 0, binding.psa_last_error()
    return d


def test_noalloc_matches_allocating_backward_twice():
    t = torch()
    big = inputs.WORKLOADS["midres_n1600_bf16"].with_(B=4)
    small = inputs.WORKLOADS["batched_n400_bf16"].with_(B=2, heads=2, H=15, W=21, seed=41)  # N = 315, ragged
    for wl in (big, small):
        x = inputs.make_inputs(wl)
        qkv, dO = device_inputs(x)
        o, lse = binding.fwd(qkv, wl.dk, wl.dv, wl.scale)
        ref = binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale)
        got = _noalloc(qkv, o, lse, dO, wl)
        t.cuda.synchronize()
        assert t.equal(got, ref), wl.name
        sl = inputs.sample_slices(wl, 2)
        d_ref = orc.backward(x.qkv, to_host(o), to_host(lse), x.dO, wl.dk, wl.dv, wl.scale, slices=sl)
        g = to_host(got).reshape(wl.BH, wl.channels, wl.N)[sl]
        r = d_ref.reshape(wl.BH, wl.channels, wl.N)[sl]
        assert np.isfinite(g).all()
        assert orc.max_rel_err(g, r) <= TOL[wl.dtype]


def test_noalloc_unpadded_rows_match_padded():
    """At N = 1599 the allocating backward stages its inputs into rows padded
    to a multiple of 8; the allocation-free one reads the ragged rows as they
    are.  Same kernels otherwise: bitwise equal."""
    t = torch()
    wl = inputs.WORKLOADS["midres_n1600_bf16"].with_(B=1, heads=2, H=41, W=39, seed=43)  # N = 1599
    x = inputs.make_inputs(wl)
    qkv, dO = device_inputs(x)
    o, lse = binding.fwd(qkv, wl.dk, wl.dv, wl.scale)
    ref = binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale)
    got = _noalloc(qkv, o, lse, dO, wl)
    t.cuda.synchronize()
    assert t.equal(got, ref)
    sl = inputs.sample_slices(wl, 1)
    d_ref = orc.backward(x.qkv, to_host(o), to_host(lse), x.dO, wl.dk, wl.dv, wl.scale, slices=sl)
    g = to_host(got).reshape(wl.BH, wl.channels, wl.N)[sl]
    assert orc.max_rel_err(g, d_ref.reshape(wl.BH, wl.channels, wl.N)[sl]) <= TOL[wl.dtype]


def test_noalloc_refuses_beyond_its_limit():
    t = torch()
    qkv = t.zeros((1, 1, 128, 8), dtype=t.bfloat16, device="cuda")
    rc = binding.psa_attn_bwd_noalloc(qkv.data_ptr(), qkv.data_ptr() + 4096, qkv.data_ptr(), qkv.data_ptr(),
                                      qkv.data_ptr(), 1024, 8, 4096, 32, 64, 0.17, binding.PSA_BF16,
                                      t.cuda.current_stream().cuda_stream)
    assert rc == 2 and "static scratch limit" in binding.psa_last_error()
