"""CPU checks of the seeded input generator (attn_inputs): bf16 rounding is
round-to-nearest-even on every class of fp32 value, and the chunked generator
does not depend on the thread count."""
import numpy as np

import attn_inputs as ai


def test_bf16_rounding_nearest_even():
    # (fp32 bit pattern, expected bf16 bit pattern)
    cases = [
        (0x3F800000, 0x3F80),  # 1.0 exact
        (0x3F808000, 0x3F80),  # halfway, even below -> stays
        (0x3F818000, 0x3F82),  # halfway, odd below -> rounds up
        (0x3F808001, 0x3F81),  # just above halfway -> up
        (0x3F807FFF, 0x3F80),  # just below halfway -> down
        (0xBF808001, 0xBF81),  # negative, magnitude rounds up
        (0x7F7FFFFF, 0x7F80),  # largest finite -> overflows to +inf
        (0xFF7FFFFF, 0xFF80),  # most negative finite -> -inf
        (0x7F800000, 0x7F80),  # +inf
        (0xFF800000, 0xFF80),  # -inf
        (0x00000001, 0x0000),  # smallest subnormal -> +0
        (0x80000000, 0x8000),  # -0
        (0x7FC00001, 0x7FC0),  # NaN -> canonical quiet NaN
        (0xFFFFFFFF, 0x7FC0),  # NaN with every bit set (the 32-bit sum would wrap)
    ]
    x = np.array([c[0] for c in cases], dtype=np.uint32).view(np.float32)
    got = ai.f32_to_bf16_bits(x)
    assert got.tolist() == [c[1] for c in cases]


def test_bf16_rounding_matches_wide_integer_form():
    rng = np.random.default_rng(5)
    x = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    ref = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    ref[np.isnan(x)] = 0x7FC0
    assert np.array_equal(ai.f32_to_bf16_bits(x), ref)


def test_chunked_generator_is_thread_count_independent():
    a = ai.make_inputs_chunked(1, 2, 1000, 64, 9, with_dout=True, threads=1)
    b = ai.make_inputs_chunked(1, 2, 1000, 64, 9, with_dout=True, threads=5)
    assert sorted(a) == ["do", "k", "q", "v"]
    for n in a:
        assert a[n].shape == (1, 2, 1000, 64) and np.array_equal(a[n], b[n])
    f = ai.bf16_bits_to_f32(a["q"])
    assert abs(float(f.mean())) < 0.02 and abs(float(f.std()) - 1.0) < 0.02
