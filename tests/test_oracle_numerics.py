"""Pins of the oracle's number-format helpers against IEEE 754 facts."""
import numpy as np

from oracle.numerics import bf16_to_f64, f64_to_fp16, fp16_to_f64


def test_bf16_decode_known_patterns():
    bits = np.array([0x0000, 0x3F80, 0xC000, 0x4049, 0x0001, 0x7F7F], dtype=np.uint16)
    want = [0.0, 1.0, -2.0, 3.140625, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127]
    assert bf16_to_f64(bits).tolist() == want


def test_fp16_single_rounding_from_f64():
    # 1 + 2^-11 is the fp16 half-way point between 1 and 1 + 2^-10.  A value just above it must
    # round up; going through binary32 first would land exactly on the half-way point and then
    # round to even (down).
    x = 1.0 + 2.0 ** -11 + 2.0 ** -40
    assert fp16_to_f64(f64_to_fp16(x)) == 1.0 + 2.0 ** -10
    assert fp16_to_f64(np.float16(np.float32(x))) == 1.0  # the double-rounding answer


def test_fp16_ties_to_even():
    assert fp16_to_f64(f64_to_fp16(1.0 + 2.0 ** -11)) == 1.0
    assert fp16_to_f64(f64_to_fp16(1.0 + 3 * 2.0 ** -11)) == 1.0 + 2 * 2.0 ** -10
    assert fp16_to_f64(f64_to_fp16(-(1.0 + 2.0 ** -11))) == -1.0


def test_fp16_subnormals_and_overflow():
    tiny = 2.0 ** -24  # smallest fp16 subnormal
    assert fp16_to_f64(f64_to_fp16(tiny)) == tiny
    assert fp16_to_f64(f64_to_fp16(0.5 * tiny)) == 0.0           # tie to even (0)
    assert fp16_to_f64(f64_to_fp16(0.75 * tiny)) == tiny
    assert fp16_to_f64(f64_to_fp16(1.5 * tiny)) == 2 * tiny       # tie to even (2)
    assert fp16_to_f64(f64_to_fp16(65504.0)) == 65504.0
    assert fp16_to_f64(f64_to_fp16(65519.99)) == 65504.0
    assert np.isinf(fp16_to_f64(f64_to_fp16(65520.0)))
