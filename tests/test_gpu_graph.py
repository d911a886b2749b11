"""fwd and bwd captured into HIP graphs (no allocation, no memset inside the
calls once the scratch buffer exists) and replayed several times, with eager
calls and synchronisations in between: every replay equals the eager result
bit for bit (the kernels are deterministic)."""
import pytest

from vision_transformer_attention_psa_amd import binding, inputs

from gpu_helpers import device_inputs, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["batched_n400_bf16", "nano_n400_f32"])
def test_graph_replays_match_eager(name):
    t = torch()
    wl = inputs.WORKLOADS[name]
    x = inputs.make_inputs(wl)
    qkv, dO = device_inputs(x)
    o_ref, l_ref = binding.fwd(qkv, wl.dk, wl.dv, wl.scale)
    d_ref = binding.bwd(qkv, o_ref, l_ref, dO, wl.dk, wl.dv, wl.scale)
    t.cuda.synchronize()

    o, lse, d = t.empty_like(o_ref), t.empty_like(l_ref), t.empty_like(d_ref)
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):  # the capture stream's scratch exists before capture
        binding.fwd(qkv, wl.dk, wl.dv, wl.scale, out=(o, lse))
        binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale, out=d)
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=s):
        binding.fwd(qkv, wl.dk, wl.dv, wl.scale, out=(o, lse))
        binding.bwd(qkv, o, lse, dO, wl.dk, wl.dv, wl.scale, out=d)
    for rep in range(4):
        for buf in (o, lse, d):
            buf.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(o, o_ref) and t.equal(lse, l_ref) and t.equal(d, d_ref), f"replay {rep}"
        # eager work on the default stream between replays
        o2, l2 = binding.fwd(qkv, wl.dk, wl.dv, wl.scale)
        d2 = binding.bwd(qkv, o2, l2, dO, wl.dk, wl.dv, wl.scale)
        t.cuda.synchronize()
        assert t.equal(d2, d_ref)
