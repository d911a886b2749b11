"""The binding refuses tensors that are not on a GPU before it calls the
library: the library receives raw addresses, and a host address handed to a
kernel is a GPU memory fault.  Runs on the CPU; the library is never called
(its loader is replaced by one that fails the test)."""
import pytest

torch = pytest.importorskip("torch")

from vision_transformer_attention_psa_amd import binding  # noqa: E402


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def forbidden(*a, **k):
        raise AssertionError("the library was called with host tensors")
    monkeypatch.setattr(binding, "load", forbidden)
    monkeypatch.setattr(binding, "_lib", None)


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


B, H, N, DK, DV = 1, 2, 16, 32, 64


def test_fwd_rejects_host_qkv():
    with pytest.raises(ValueError, match="qkv is on cpu"):
        binding.fwd(t(B, H, 2 * DK + DV, N), DK, DV, 0.2)


def test_fwd_rejects_host_outputs():
    with pytest.raises(ValueError, match="on cpu"):
        binding.fwd(t(B, H, 2 * DK + DV, N), DK, DV, 0.2,
                    out=(t(B, H, DV, N), t(B, H, N, dtype=torch.float32)))


def test_bwd_rejects_host_tensors():
    with pytest.raises(ValueError, match="on cpu"):
        binding.bwd(t(B, H, 2 * DK + DV, N), t(B, H, DV, N), t(B, H, N, dtype=torch.float32),
                    t(B, H, DV, N), DK, DV, 0.2)


def test_vslice_calls_reject_host_tensors():
    qkv = t(B, H, 2 * DK + DV, N)
    with pytest.raises(ValueError, match="on cpu"):
        binding.fwd_vslice(qkv, DK, DV, 0, DV // 2, 0.2)
    with pytest.raises(ValueError, match="on cpu"):
        binding.bwd_vslice(qkv, t(B, H, DV // 2, N), t(B, H, N, dtype=torch.float32), t(B, H, DV // 2, N),
                           t(B, H, 2 * DK + DV, N), DK, DV, 0, DV // 2, 0.2, accumulate=False)


def test_merge_rejects_host_tensors():
    with pytest.raises(ValueError, match="on cpu"):
        binding.merge_fwd(t(B, H, 8, N), t(B, H, 8, N))
    with pytest.raises(ValueError, match="on cpu"):
        binding.merge_bwd(t(B, H, 16, N))


def test_conv_and_cat_reject_host_tensors():
    x, w, dy = t(2, 128, N), t(256, 128), t(2, 256, N)
    with pytest.raises(ValueError, match="on cpu"):
        binding.conv_bwd(x, w, dy)
    with pytest.raises(ValueError, match="on cpu"):
        binding.conv_cat_bwd(x, w, dy, [64, 64])
    with pytest.raises(ValueError, match="on cpu"):
        binding.channel_cat_bwd(t(2, 8, 4, 4), 4, 4)


class FakeGpuTensor:
    """Stands in for a tensor on a given GPU (only what the check reads)."""

    def __init__(self, index):
        self.is_cuda = True
        self.device = torch.device("cuda", index)


def test_mixed_devices_rejected():
    binding._on_gpu("fwd", ("qkv", FakeGpuTensor(0)), ("o", FakeGpuTensor(0)))
    with pytest.raises(ValueError, match="one GPU"):
        binding._on_gpu("bwd", ("qkv", FakeGpuTensor(0)), ("dO", FakeGpuTensor(1)))
