"""Host-side checks of the seeded workload generator (no GPU, no oracle)."""
import numpy as np

from vision_transformer_attention_psa_amd import inputs


def test_bf16_round_to_nearest_even_bit_patterns():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -7 + 2.0 ** -9,
                  -2.5, 0.0, -0.0, 3.4e38, np.inf, -np.inf, 1.0e-40], dtype=np.float32)
    bits = inputs.bf16_bits_rne(x)
    # 1 + 2^-8 is a tie between 0x3F80 and 0x3F81 -> even (0x3F80);
    # 1 + 3*2^-8 is a tie between 0x3F81 and 0x3F82 -> even (0x3F82);
    # 1 + 2^-7 + 2^-9 is below the halfway point -> 0x3F81; 3.4e38 lies past
    # the midpoint between the largest bf16 and 2^128 -> +inf.
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000, 0x8000,
                             0x7F80, 0x7F80, 0xFF80, 0x0001]
    back = inputs.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[4] == -2.5 and np.isinf(back[7])
    nan = inputs.bf16_bits_rne(np.array([np.nan], dtype=np.float32))
    assert np.isnan(inputs.bf16_bits_to_f32(nan))[0]


def test_bf16_rounding_error_bound():
    rng = np.random.Generator(np.random.PCG64(7))
    x = rng.standard_normal(100000).astype(np.float32)
    y = inputs.bf16_bits_to_f32(inputs.bf16_bits_rne(x))
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)


def test_workload_shapes_and_determinism():
    for name, wl in inputs.WORKLOADS.items():
        small = wl.with_(B=1, heads=1) if wl.N > 400 else wl
        a, b = inputs.make_inputs(small), inputs.make_inputs(small)
        assert a.qkv.shape == (small.B, small.heads, 2 * wl.dk + wl.dv, wl.N)
        assert a.dO.shape == (small.B, small.heads, wl.dv, wl.N)
        np.testing.assert_array_equal(a.qkv, b.qkv)
        if wl.dtype == inputs.BF16:
            np.testing.assert_array_equal(inputs.bf16_bits_to_f32(a.qkv_bits), a.qkv)


def test_f16_rounding_is_ieee_rne():
    """binary16 patterns of values whose rounding is fixed by IEEE 754:
    exact values, ties to even, overflow and the smallest subnormal."""
    vals = np.array([1.0, -2.0, 65504.0, 65519.0, 65520.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11,
                     2.0 ** -24, 2.0 ** -26, 0.1], dtype=np.float32)
    want = [0x3C00, 0xC000, 0x7BFF, 0x7BFF, 0x7C00, 0x3C00, 0x3C02, 0x0001, 0x0000, 0x2E66]
    assert inputs.f16_bits_rne(vals).tolist() == want
    back = inputs.f16_bits_to_f32(np.array(want, dtype=np.uint16))
    assert back[0] == 1.0 and back[2] == 65504.0 and np.isinf(back[4]) and back[7] == 2.0 ** -24


def test_f16_workload_values_are_representable():
    wl = inputs.WORKLOADS["batched_n400_bf16"].with_(B=1, dtype=inputs.F16)
    x = inputs.make_inputs(wl)
    np.testing.assert_array_equal(inputs.f16_bits_to_f32(x.qkv_bits), x.qkv)
    np.testing.assert_array_equal(x.qkv.astype(np.float16).astype(np.float32), x.qkv)


def test_highres_qk_sigma():
    wl = inputs.WORKLOADS["highres_n6400_bf16"].with_(B=1, heads=1)
    x = inputs.make_inputs(wl)
    qk = x.qkv[0, 0, : 2 * wl.dk]
    v = x.qkv[0, 0, 2 * wl.dk:]
    assert 2.9 < qk.std() < 3.1 and 0.97 < v.std() < 1.03


def test_sample_slices():
    wl = inputs.WORKLOADS["midres_n1600_bf16"]
    s = inputs.sample_slices(wl, 4)
    assert s[0] == 0 and s[-1] == wl.BH - 1 and len(s) == 4
    assert inputs.sample_slices(wl, 4) == s
    assert inputs.sample_slices(wl, 1000) == list(range(wl.BH))
