"""The seeded input generator (CPU only)."""
import numpy as np

import gen


def test_philox_known_answers():
    # Known-answer vectors of Philox-4x32-10 published with the Random123
    # library (Salmon et al., SC'11): zero, all-ones, and pi-digit inputs.
    assert gen.philox4x32_10([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert gen.philox4x32_10([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert gen.philox4x32_10([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0]) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_stream_prefix_and_offsets():
    a = gen.normal(0, 1, (1001,), 1.0, gen.F32)
    for begin, n in ((0, 1), (1, 1), (3, 10), (500, 501)):
        assert np.array_equal(gen.normal(0, 1, (n,), 1.0, gen.F32, begin=begin), a[begin:begin + n])
    assert not np.array_equal(gen.normal(0, 2, (1001,), 1.0, gen.F32), a)
    assert not np.array_equal(gen.normal(1, 1, (1001,), 1.0, gen.F32), a)


def test_moments():
    a = gen.normal(0, 7, (2_000_000,), 0.5, gen.F32).astype(np.float64)
    assert abs(a.mean()) < 0.002 and abs(a.std() - 0.5) < 0.002
    # standard-normal tail mass beyond 3 sigma is 0.0027
    assert abs((np.abs(a) > 1.5).mean() - 0.0027) < 0.0003


def test_bf16_is_rounded_fp32():
    f = gen.normal(3, 4, (100_000,), 2.0, gen.F32)
    b = gen.normal(3, 4, (100_000,), 2.0, gen.BF16)
    assert np.array_equal(gen.f32_to_bf16_bits(f), b)
    bf = gen.bf16_bits_to_f32(b)
    # round-to-nearest: error at most half a bf16 ulp
    ulp = np.exp2(np.floor(np.log2(np.abs(f))) - 7)
    assert np.all(np.abs(bf - f) <= ulp / 2)
    # ties go to even
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float32)
    assert gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(ties)).tolist() == [1.0, 1 + 2 ** -6]


def test_config_shapes():
    cfg = gen.CONFIGS["tiny"]
    w = gen.make_all(cfg, 32)
    assert w["x"].shape == (32, 64) and w["x"].dtype == np.float32
    assert w["w1"].shape == (4, 64, 128) and w["w2"].shape == (4, 128, 64)
    assert w["b1"].shape == (4, 128) and w["b2"].shape == (4, 64) and w["w3"] is None
    assert w["b_r"] is None
    b = gen.router_bias(gen.CONFIGS["skew16"])
    assert b.shape == (16,) and b.dtype == np.float32
