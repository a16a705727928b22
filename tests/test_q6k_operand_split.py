"""The Q6_K MMQ's operand split, on the host: for every int8 scale sc and
6-bit code q, u = -sc*(q-32) = 32*a + b with int8 a and b in [0, 31], formed
the way the kernel forms it (16-bit lanes: u = q*(-sc) + 32*sc modulo 2^16,
a = u >> 5 arithmetically, b = u & 31), and the largest 32-value dot stays
below 2^24 so its f32 conversion is exact.  The Q6_K weight is
d*sc*(q-32) (Q6_K format: 16 int8 scales per 256 values, 6-bit codes with
offset 32)."""
import numpy as np


def test_split_is_exact_for_every_scale_and_code():
    q = np.arange(64, dtype=np.int64)
    for sc in range(-128, 128):
        u16 = (q * ((-sc) & 0xFFFF) + ((32 * sc) & 0xFFFF)) & 0xFFFF
        u = np.where(u16 >= 0x8000, u16 - 0x10000, u16)          # int16 lane value
        a = u >> 5                                                 # arithmetic shift
        a8 = ((a & 0xFF) ^ 0x80) - 0x80                            # low byte as int8
        b = u16 & 31
        assert np.array_equal(a8, a), sc                           # a fits int8 exactly
        assert np.array_equal(32 * a8 + b, -sc * (q - 32)), sc
        assert a8.min() >= -128 and a8.max() <= 127 and b.min() >= 0 and b.max() <= 31


def test_largest_block_dot_is_exact_in_f32():
    t = 32 * 4096 * 127                 # 32 values of |sc*(q-32)| <= 4096 times |code| <= 127
    assert t < 2 ** 24
    assert float(np.float32(t)) == t and float(np.float32(-t)) == -t
