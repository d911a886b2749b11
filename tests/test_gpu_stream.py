"""The binding launches on torch's current stream: the handle it passes is the
current stream's inside and outside a side-stream context, and a forward +
backward issued on a side stream gives the same bits as on the default
stream."""
import pytest

from vision_transformer_attention_psa_amd import binding, inputs

from gpu_helpers import device_inputs, torch

pytestmark = pytest.mark.gpu


def test_stream_handle_is_current_stream():
    t = torch()
    x = t.zeros(8, device="cuda")
    assert binding._stream(x) == t.cuda.current_stream().cuda_stream
    s = t.cuda.Stream()
    with t.cuda.stream(s):
        assert binding._stream(x) == s.cuda_stream
    assert binding._stream(x) == t.cuda.current_stream().cuda_stream


def test_side_stream_results_match_default_stream():
    t = torch()
    wl = inputs.WORKLOADS["batched_n400_bf16"].with_(B=2)
    x = inputs.make_inputs(wl)
    qkv, dO = device_inputs(x)
    o, lse = binding.fwd(qkv, wl.dk, wl.dv, wl.scale)
    d = binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale)
    t.cuda.synchronize()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        q2 = qkv.clone()  # produced on the side stream, consumed there
        o2, lse2 = binding.fwd(q2, wl.dk, wl.dv, wl.scale)
        d2 = binding.bwd(q2, o2, lse2, dO, wl.dk, wl.dv, wl.scale)
    s.synchronize()
    assert t.equal(o, o2) and t.equal(lse, lse2) and t.equal(d, d2)
