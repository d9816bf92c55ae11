"""Pins for the seeded input generator (it carries no layer arithmetic)."""
import numpy as np

import synth
from synth import DT_BF16, DT_F32


def test_splitmix64_reference_sequence():
    # First outputs of the published splitmix64 generator seeded with 0
    # (Steele, Lea and Flood 2014; Vigna's reference C implementation).
    assert synth.splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_slices_agree():
    full = synth.normal(4, (10001,), 1.0, -1)
    for off in (0, 1, 2, 777, 9999):
        part = synth.normal(4, (10001 - off,), 1.0, -1, offset=off)
        assert np.array_equal(part, full[off:])
    assert synth.normal_scalar(4, 1234) == full[1234]


def test_normal_moments_and_streams_independent():
    x = synth.normal(1, (1 << 20,), 1.0, -1)
    y = synth.normal(2, (1 << 20,), 1.0, -1)
    assert abs(x.mean()) < 5e-3 and abs(x.var() - 1) < 1e-2
    assert abs(np.corrcoef(x, y)[0, 1]) < 5e-3
    assert abs(np.corrcoef(x[0::2], x[1::2])[0, 1]) < 5e-3   # the two Box-Muller branches


def test_bf16_round_to_nearest_even():
    one = 1.0
    vals = np.array([one, one + 2.0 ** -8, one + 3 * 2.0 ** -8, one + 2.0 ** -8 + 2.0 ** -20, -2.5,
                     3.0e38], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(vals)
    # halfway cases go to the even neighbour; just above halfway rounds up; 3e38 stays finite
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F62]
    assert np.array_equal(synth.bf16_bits_to_f32(bits[:2]), np.array([1.0, 1.0], dtype=np.float32))


def test_bf16_fill_equals_rounded_fp32_fill():
    a = synth.normal(5, (4096,), 0.3, DT_F32)
    b = synth.normal(5, (4096,), 0.3, DT_BF16)
    assert np.array_equal(synth.f32_to_bf16_bits(a), b)


def test_decode_tokens_are_prefill_prefix():
    p, d = synth.WORKLOADS["c4p"], synth.WORKLOADS["c4d"]
    up = synth.normal(synth.STREAM_U, (256, p.H), 1.0, DT_BF16)
    ud = synth.make_inputs(d, weights=False)["u"]
    assert np.array_equal(ud, up[:d.T])


def test_recipe_scales():
    c2 = synth.WORKLOADS["c2"]
    s = synth.centroid_row_scale(c2)
    assert np.array_equal(s[:8], np.full(8, 1.5)) and np.array_equal(s[8:], np.ones(c2.N_r - 8))
    c4 = synth.WORKLOADS["c4p"]
    z = synth.centroid_row_scale(c4)
    assert abs(np.mean(z * z) - 1.0) < 1e-12
    assert sorted(synth.permutation(synth.STREAM_ZIPF_PERM, c4.N_r).tolist()) == list(range(c4.N_r))
    assert z.max() / z.min() > 20.0   # norms span far more than 20x
