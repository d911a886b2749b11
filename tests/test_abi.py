"""The C ABI library loads, exports every symbol the header declares, and
rejects bad arguments before touching the GPU (no compute call here)."""
import ctypes
import os
import re

import pytest

from vision_transformer_attention_psa_amd import binding
from vision_transformer_attention_psa_amd.build import LIB_PATH, ROOT

HEADER = os.path.join(ROOT, "include", "psa_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        pytest.fail(f"{LIB_PATH} not built; run __graft_entry__.build() first")
    return binding.load()


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_supported_table(lib):
    F32, BF16, F16 = binding.PSA_F32, binding.PSA_BF16, binding.PSA_F16
    for dk, dv in [(16, 16), (32, 32), (32, 64), (64, 32), (64, 64), (64, 128), (128, 128)]:
        assert binding.psa_attn_supported(dk, dv, F32)
    for dk, dv in [(32, 32), (32, 64), (64, 32), (64, 64), (64, 128), (128, 128)]:
        assert binding.psa_attn_supported(dk, dv, BF16)
        assert binding.psa_attn_supported(dk, dv, F16)
    assert not binding.psa_attn_supported(128, 64, BF16)
    assert not binding.psa_attn_supported(16, 16, BF16)
    assert not binding.psa_attn_supported(16, 16, F16)
    assert not binding.psa_attn_supported(48, 64, F32)
    assert not binding.psa_attn_supported(32, 64, 7)
    assert binding.psa_attn_version() >= 100


A = 1 << 20  # fake, 16-byte aligned, non-overlapping addresses: validation
B_ = 1 << 30  # fails before any of them is dereferenced


@pytest.mark.parametrize("args,code,needle", [
    (dict(qkv=0), 1, "non-NULL"),
    (dict(N=0), 2, ">= 1"),
    (dict(B=-1), 2, ">= 1"),
    (dict(scale=0.0), 2, "scale"),
    (dict(scale=float("nan")), 2, "scale"),
    (dict(dk=48), 3, "no compiled instance"),
    (dict(dtype=5), 3, "dtype"),
    (dict(o=A + 8), 4, "aligned"),
    (dict(o=A + 64), 5, "overlap"),
])
def test_fwd_validation(lib, args, code, needle):
    kw = dict(qkv=A, o=B_, lse=B_ * 2, B=2, heads=2, N=100, dk=32, dv=64, scale=0.17,
              dtype=binding.PSA_BF16, stream=None)
    kw.update(args)
    rc = binding.psa_attn_fwd(**kw)
    assert rc == code
    assert needle in binding.psa_last_error()


@pytest.mark.parametrize("args,code,needle", [
    (dict(dO=0), 1, "non-NULL"),
    (dict(heads=0), 2, ">= 1"),
    (dict(dv=48), 3, "no compiled instance"),
    (dict(lse=B_ * 3 + 4), 4, "aligned"),
    (dict(d_packed=A), 5, "overlap"),
    (dict(d_packed=B_ * 2 - 16), 5, "overlap"),
])
def test_bwd_validation(lib, args, code, needle):
    kw = dict(qkv=A, o=B_, lse=B_ * 3, dO=B_ * 2, d_packed=B_ * 4, B=2, heads=2, N=100, dk=32,
              dv=64, scale=0.17, dtype=binding.PSA_BF16, stream=None)
    kw.update(args)
    rc = binding.psa_attn_bwd(**kw)
    assert rc == code
    assert needle in binding.psa_last_error()


def test_huge_problem_rejected(lib):
    rc = binding.psa_attn_fwd(A, B_, B_ * 2, 1 << 20, 1 << 10, 1 << 20, 32, 64, 0.1,
                              binding.PSA_BF16, None)
    assert rc == 2 and "too large" in binding.psa_last_error()


def test_noalloc_limit_rejected_before_any_device_call(lib):
    """B*heads*N beyond the static scratch (2^21 queries) is refused with
    PSA_ERR_SHAPE from the arguments alone (fake addresses, no GPU)."""
    kw = dict(qkv=A, o=B_, lse=B_ * 3, dO=B_ * 2, d_packed=B_ * 4, B=64, heads=8, N=4097, dk=32,
              dv=64, scale=0.17, dtype=binding.PSA_BF16, stream=None)
    assert 64 * 8 * 4097 > 1 << 21
    rc = binding.psa_attn_bwd_noalloc(**kw)
    assert rc == 2
    assert "static scratch limit of 2097152" in binding.psa_last_error()
