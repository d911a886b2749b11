"""torch autograd through the C ABI: O from psa_attention, and qkv.grad from
loss.backward() equal to psa_attn_bwd's d_packed bit for bit and to the
oracle within the bar."""
import numpy as np
import pytest

from oracle import psa_oracle as orc
from vision_transformer_attention_psa_amd import binding, inputs

from gpu_helpers import TOL, device_inputs, to_host, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["nano_n400_f32", "batched_n400_bf16"])
def test_autograd_matches_bwd_and_oracle(name):
    t = torch()
    wl = inputs.WORKLOADS[name]
    x = inputs.make_inputs(wl)
    qkv, dO = device_inputs(x)
    leaf = qkv.clone().requires_grad_(True)
    o = binding.psa_attention(leaf, wl.dk, wl.dv, wl.scale)
    o.backward(dO)
    t.cuda.synchronize()
    o2, lse2 = binding.fwd(qkv, wl.dk, wl.dv, wl.scale)
    d2 = binding.bwd(qkv, o2, lse2, dO, wl.dk, wl.dv, wl.scale)
    t.cuda.synchronize()
    assert t.equal(o.detach(), o2) and t.equal(leaf.grad, d2)
    ro, _, rd = orc.forward_backward(x.qkv, x.dO, wl.dk, wl.dv, wl.scale)
    assert orc.max_rel_err(to_host(o.detach()), ro) <= TOL[wl.dtype]
    assert orc.max_rel_err(to_host(leaf.grad), rd) <= TOL[wl.dtype]
    assert np.isfinite(to_host(leaf.grad)).all()
