"""The seeded generator: determinism, value ranges, storage formats."""

import numpy as np

import synth


def test_seed_determinism_and_weight_sharing_across_M():
    a = synth.make_inputs(4, 1, 256, 64, 128, seed=(7, 1))
    b = synth.make_inputs(4, 1, 256, 64, 128, seed=(7, 1))
    c = synth.make_inputs(4, 8, 256, 64, 128, seed=(7, 1))
    for f in ("qweight", "qzeros", "scales", "x"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert np.array_equal(a.qweight, c.qweight) and np.array_equal(a.scales, c.scales)


def test_value_ranges_w4():
    c = synth.make_inputs(4, 2, 512, 128, 128, seed=(8,))
    assert c.codes.max() <= 15 and c.zeros.max() <= 15
    s = synth.bf16_bits_to_f32(c.scales)
    assert s.min() >= 0.002 - 1e-5 and s.max() < 0.2
    assert c.qweight.dtype == np.uint32 and c.qweight.shape == (512, 16)


def test_value_ranges_w8():
    c = synth.make_inputs(8, 1, 256, 64, 256, seed=(9,))
    assert c.zeros.min() >= 112 and c.zeros.max() <= 143
    s = synth.bf16_bits_to_f32(c.scales)
    assert s.min() >= 0.0005 - 1e-6 and s.max() < 0.05


def test_outlier_channels():
    c = synth.make_inputs(4, 64, 4096, 8, 128, seed=(10,), outlier_frac=0.01)
    x = synth.bf16_bits_to_f32(c.x)
    big = np.abs(x).max(axis=0) > 8.0
    assert 30 <= big.sum() <= 41


def test_bf16_helpers_roundtrip():
    rng = np.random.default_rng(0)
    f = rng.standard_normal(1000).astype(np.float32)
    b = synth.f32_to_bf16_bits(f)
    assert np.array_equal(synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(b)), b)
    assert np.all(np.abs(synth.bf16_bits_to_f32(b) - f) <= np.abs(f) * 2**-8)


def test_configs_table():
    assert synth.CONFIGS[1]["Ms"] == (1, 4, 8)
    assert len(synth.CONFIGS[1]["shapes"]) == 7
    c = synth.make_case(0, 0, 1, keep_codes=False)
    assert (c.K, c.N, c.G, c.bits) == (4096, 4096, 128, 4)
