"""The C ABI refuses memory that is not device memory of the current device,
before anything is enqueued.  The host buffer here is pinned (hipHostMalloc
through torch), which the GPU can address: had the check let it through, the
kernel would still read valid memory, so the test cannot fault the GPU."""
import pytest

from vision_transformer_attention_psa_amd import binding

from gpu_helpers import torch

pytestmark = pytest.mark.gpu


def test_pinned_host_output_refused():
    t = torch()
    B, H, N, dk, dv = 1, 1, 64, 32, 64
    qkv = t.zeros((B, H, 2 * dk + dv, N), dtype=t.bfloat16, device="cuda")
    lse = t.empty((B, H, N), dtype=t.float32, device="cuda")
    o_host = t.full((B, H, dv, N), 3.0, dtype=t.bfloat16).pin_memory()
    rc = binding.psa_attn_fwd(qkv.data_ptr(), o_host.data_ptr(), lse.data_ptr(), B, H, N, dk, dv, 0.17,
                              binding.PSA_BF16, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    assert rc == 8, (rc, binding.psa_last_error())
    assert "o is not device memory" in binding.psa_last_error()
    assert (o_host.float() == 3.0).all()  # nothing was written


def test_binding_refuses_pinned_host_tensor():
    t = torch()
    qkv = t.zeros((1, 1, 128, 64), dtype=t.bfloat16).pin_memory()
    with pytest.raises(ValueError, match="on cpu"):
        binding.fwd(qkv, 32, 64, 0.17)


def test_device_memory_accepted_after_a_refusal():
    """A refused call leaves no HIP error behind for the next launch."""
    t = torch()
    B, H, N, dk, dv = 1, 2, 96, 32, 64
    qkv = t.randn((B, H, 2 * dk + dv, N), device="cuda").to(t.bfloat16)
    bad = t.empty((B, H, dv, N), dtype=t.bfloat16).pin_memory()
    lse = t.empty((B, H, N), dtype=t.float32, device="cuda")
    rc = binding.psa_attn_fwd(qkv.data_ptr(), bad.data_ptr(), lse.data_ptr(), B, H, N, dk, dv, 0.17,
                              binding.PSA_BF16, t.cuda.current_stream().cuda_stream)
    assert rc == 8
    o, lse2 = binding.fwd(qkv, dk, dv, 0.17)
    t.cuda.synchronize()
    assert t.isfinite(o.float()).all() and t.isfinite(lse2).all()
