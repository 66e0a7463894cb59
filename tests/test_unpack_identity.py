"""CPU pin of the packed-fp16 floor-by-3 identity the GPU kernels unpack with.

The kernels hold a byte v (0..242) as the fp16 value 1024 + v and compute one
fused multiply-add (1024 + v) * M + A, rounded to fp16 (round to nearest,
ties to even).  In [1024, 2048) fp16 values are the integers, so the identity
claimed in ternary_matvec_amd/csrc/unpack.hpp is that the rounded result is
exactly 1024 + floor(v / 3) for every v, and that chaining it yields
floor(v / 9), floor(v / 27) and floor(v / 81).  The constants M and A are read
from that source file, so a change there is checked here.  The fused product
is formed exactly with rationals and rounded once, as the FMA does.
"""
import os
import re
from fractions import Fraction

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "ternary_matvec_amd", "csrc", "unpack.hpp")


def fp16_value(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 10) & 0x1F
    frac = bits & 0x3FF
    assert exp not in (0, 31), "only normal fp16 constants are expected"
    return sign * Fraction(1024 + frac, 1024) * Fraction(2) ** (exp - 15)


def round_fp16(x: Fraction) -> Fraction:
    """Round a positive value in fp16's normal range to the nearest fp16 value, ties to even."""
    assert Fraction(2) ** -14 <= x < 65504
    e = 0
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    while Fraction(2) ** e > x:
        e -= 1
    ulp = Fraction(2) ** (e - 10)
    return round(x / ulp) * ulp        # Fraction.__round__ rounds half to even


def constants():
    src = open(SRC).read()
    body = src[src.index("third2"):]
    mul = re.search(r"mul\s*=\s*__builtin_bit_cast\(half2_t,\s*0x([0-9a-fA-F]{8})u\)", body).group(1)
    add = re.search(r"add\s*=\s*__builtin_bit_cast\(half2_t,\s*0x([0-9a-fA-F]{8})u\)", body).group(1)
    m, a = int(mul, 16), int(add, 16)
    assert m >> 16 == m & 0xFFFF and a >> 16 == a & 0xFFFF, "both fp16 lanes use the same constant"
    return fp16_value(m & 0xFFFF), fp16_value(a & 0xFFFF)


def third(h: int, mul: Fraction, add: Fraction) -> Fraction:
    return round_fp16(h * mul + add)


def test_constants_are_the_documented_values():
    mul, add = constants()
    assert mul == Fraction(0.332763671875) and add == 683


@pytest.mark.parametrize("v", range(243))
def test_floor_by_three_chain_for_every_byte_code(v):
    mul, add = constants()
    h = 1024 + v
    for d in (3, 9, 27, 81):
        h = third(h, mul, add)
        assert h == 1024 + v // d, (v, d, h)
    # the fp16 bit pattern of 1024 + p is 0x6400 + p: its low byte is p
    assert (0x6400 + v // 81) & 0xFF == v // 81


def test_identity_fails_for_a_wrong_constant():
    # the check above is sensitive: one fp16 step off in either constant breaks it
    mul, add = constants()
    step_mul = Fraction(1, 2 ** 12)      # fp16 ulp in [0.25, 0.5)
    for m2, a2 in ((mul + step_mul, add), (mul - step_mul, add), (mul, add + 1), (mul, add - 1)):
        bad = [v for v in range(243) if third(1024 + v, m2, a2) != 1024 + v // 3]
        assert bad, (m2, a2)
