"""Parity of the 1x1-convolution backward (psa_qkv_conv_bwd, through the C
ABI) against the float64 oracle, at the same per-tensor bars as the
attention: max|gpu - ref| / max|ref| over dx and over dw."""
import numpy as np
import pytest

from oracle import conv_oracle as co
from oracle import psa_oracle as orc
from vision_transformer_attention_psa_amd import binding, inputs

from gpu_helpers import TOL, device_inputs, run_chained, to_device, to_host, torch

pytestmark = pytest.mark.gpu

SHAPES = [
    # (dtype, B, cin, cout, N)
    (inputs.F32, 1, 128, 128, 1),
    (inputs.F32, 2, 128, 384, 97),
    (inputs.BF16, 2, 128, 384, 97),
    (inputs.BF16, 3, 128, 256, 1003),
    (inputs.F16, 1, 256, 512, 400),
    (inputs.BF16, 16, 256, 512, 400),   # the N = 400 attention block's projection
    (inputs.BF16, 8, 512, 1024, 1600),  # the N = 1600 block
    (inputs.BF16, 4, 512, 1536, 6400),  # the N = 6400 block
    (inputs.F16, 4, 512, 1536, 6400),
    # large-tile dx pipeline: a partial last token tile; N not a multiple
    # of 8 (rows staged into zero-padded copies, remainders 7 and 5); cin
    # not a multiple of 256 (128 x 256 tiles)
    (inputs.BF16, 4, 512, 1024, 6000),
    (inputs.BF16, 4, 512, 1536, 6399),
    (inputs.F16, 4, 384, 512, 6400),
    (inputs.BF16, 4, 384, 512, 6397),
    # large-tile dw pipeline (cin a multiple of 256): a last token stage of
    # 48 and of 8 tokens (the upper half-stage all past the row end), and
    # rows padded to 1008 with a 48-token last stage
    (inputs.F16, 4, 512, 1024, 6408),
    (inputs.F16, 8, 512, 1024, 1001),
    # 192 tiles fill the CUs on their own: one range, dw written directly
    (inputs.BF16, 1, 4096, 1536, 200),
]


def _device(ci):
    return tuple(to_device(a, None if ci.bits is None else ci.bits[k], ci.dtype)
                 for k, a in enumerate((ci.x, ci.w, ci.dy)))


def run_conv(ci):
    x, w, dy = _device(ci)
    dx, dw = binding.conv_bwd(x, w, dy)
    torch().cuda.synchronize()
    return to_host(dx), to_host(dw)


@pytest.mark.parametrize("dtype,B,cin,cout,N", SHAPES)
def test_conv_backward_parity(dtype, B, cin, cout, N):
    ci = inputs.make_conv_inputs(B, cin, cout, N, dtype, seed=500 + N + cin)
    dx, dw = run_conv(ci)
    rdx, rdw = co.conv1x1_backward(ci.x, ci.w, ci.dy)
    e = {"dx": orc.max_rel_err(dx, rdx), "dw": orc.max_rel_err(dw, rdw)}
    print(f"conv {dtype} B={B} cin={cin} cout={cout} N={N}", {k: f"{v:.2e}" for k, v in e.items()}, flush=True)
    assert np.isfinite(dx).all() and np.isfinite(dw).all()
    assert max(e.values()) <= TOL[dtype], e


@pytest.mark.parametrize("B,cin,cout,N", [(4, 256, 512, 1000), (4, 512, 1536, 6400)])
def test_conv_backward_deterministic(B, cin, cout, N):
    ci = inputs.make_conv_inputs(B, cin, cout, N, inputs.BF16, seed=3)
    a, b = run_conv(ci), run_conv(ci)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_conv_backward_of_the_attention_gradient():
    """The packed gradient psa_attn_bwd writes, fed straight to the
    projection's backward: [B, heads, 2dk+dv, N] read as [B, cout, N]."""
    wl = inputs.WORKLOADS["batched_n400_bf16"]
    x = inputs.make_inputs(wl)
    _, _, d = run_chained(x)
    cout, cin = wl.heads * wl.channels, wl.heads * wl.dv
    ci = inputs.make_conv_inputs(wl.B, cin, cout, wl.N, wl.dtype, seed=41)
    t = torch()
    xd, wd, _ = _device(ci)
    dbits = inputs.bf16_bits_rne(d.astype(np.float32))
    dyd = t.from_numpy(dbits.view(np.int16)).view(t.bfloat16).cuda()
    dx, dw = binding.conv_bwd(xd, wd, dyd)
    t.cuda.synchronize()
    rdx, rdw = co.conv1x1_backward(ci.x, ci.w, inputs.bf16_bits_to_f32(dbits))
    assert orc.max_rel_err(to_host(dx), rdx) <= TOL[wl.dtype]
    assert orc.max_rel_err(to_host(dw), rdw) <= TOL[wl.dtype]


def test_conv_backward_rejects_untiled_channels():
    ci = inputs.make_conv_inputs(1, 96, 128, 16, inputs.BF16, seed=1)
    x, w, dy = _device(ci)
    with pytest.raises(binding.PsaError, match="multiples of 128"):
        binding.conv_bwd(x, w, dy)
