"""Host-side checks of the seeded input generator (no layer arithmetic lives there)."""
import numpy as np

from lora_dora_linear_amd import inputs


def test_bf16_rounding_is_nearest_even():
    f = np.array([0x3F800000, 0x3F808000, 0x3F818000, 0x3F80FFFF, 0xBF7FFFFF], np.uint32).view(np.float32)
    np.testing.assert_array_equal(inputs.f32_to_bf16_bits(f), [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF80])
    back = inputs.bf16_bits_to_f32(np.array([0x3F80, 0xC000], np.uint16))
    np.testing.assert_array_equal(back, [1.0, -2.0])


def test_draws_are_seeded_and_shaped():
    a = inputs.linear_case(2, 33, 64, 128, 16, 0.5, "bf16")
    b = inputs.linear_case(2, 33, 64, 128, 16, 0.5, "bf16")
    for k in ("X", "W0", "A", "B", "dY"):
        np.testing.assert_array_equal(a.t[k], b.t[k])
    assert a.t["X"].shape == (33, 128) and a.t["B"].shape == (64, 16)
    x = a.f64("X")
    assert abs(x.std() - 1.0) < 0.05
    assert abs(a.f64("B").std() - np.sqrt(0.02)) < 0.02
