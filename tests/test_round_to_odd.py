"""The fp64 -> bf16 rounding the RMSNorm kernel performs, checked on the CPU.

The kernel rounds each fp64 product once to bf16 (nearest, ties to even) by
way of round-to-odd fp32: it takes the hardware's nearest-even fp32
conversion, steps one encoding toward zero where that value lies beyond the
input, and marks an inexact result in the last bit; rounding that fp32 to
bf16 is then correct (Boldo and Melquiond, "When double rounding is odd").
This test writes the same steps with numpy's nearest-even fp32 cast and
compares them with bf16 rounding computed exactly from rationals, on random
values, near-ties at both rounding steps, subnormals and overflow.  The GPU
tests compare the kernel's own output with the oracle's once-rounded value.
"""
import struct
from fractions import Fraction

import numpy as np


def derived_bf16(v: float) -> int:
    if v != v:
        return 0x7FC0
    with np.errstate(over="ignore"):
        f = np.float32(v)
    back = float(f)
    b = int(np.frombuffer(f.tobytes(), np.uint32)[0])
    if back != v:
        if abs(back) > abs(v):
            b = (b - 1) & 0xFFFFFFFF
        b |= 1
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFFFFFF
    return b >> 16


def exact_bf16(v: float) -> int:
    """bf16 (8 significant bits, fp32's exponent range) nearest to v, ties to even."""
    sign = 0x8000 if struct.pack(">d", v)[0] & 0x80 else 0
    a = Fraction(abs(v))
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = Fraction(2) ** (max(e, -126) - 7)  # spacing of bf16 values around a
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * q
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    if val < Fraction(2) ** -126:
        return sign | int(val / Fraction(2) ** -133)
    e2 = val.numerator.bit_length() - val.denominator.bit_length()
    if Fraction(2) ** e2 > val:
        e2 -= 1
    return sign | ((e2 + 127) << 7) | (int(val / Fraction(2) ** (e2 - 7)) - 128)


def test_exact_reference_known_values():
    assert exact_bf16(1.0) == 0x3F80
    assert exact_bf16(-2.0) == 0xC000
    assert exact_bf16(1.0 + 2.0 ** -8) == 0x3F80  # tie to even
    assert exact_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82  # tie to even, upward
    assert exact_bf16(1e39) == 0x7F80
    assert exact_bf16(2.0 ** -133) == 0x0001


def test_round_to_odd_derivation_matches_exact_rounding():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(4000) * 10.0 ** rng.integers(-45, 40, 4000))
    for _ in range(3000):
        m = int(rng.integers(1 << 7, 1 << 8))
        ex = int(rng.integers(-140, 130))
        base = (m + 0.5) * 2.0 ** (ex - 7)  # a bf16 rounding midpoint
        for dlt in (0.0, 2.0 ** (ex - 40), -(2.0 ** (ex - 40)), 2.0 ** (ex - 31), -(2.0 ** (ex - 31))):
            vals += [base + dlt, -(base + dlt)]
    vals += [0.0, -0.0, 3.4028235677973366e38, 3.39e38, 1e39, -1e39, 1.1754943508222875e-38, 1.17e-38,
             1e-45, 7e-46, 5e-324, 2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134]
    bad = [v for v in vals if derived_bf16(v) != exact_bf16(v)]
    assert not bad, bad[:5]
