"""CPU pin of the multiply-instead-of-divide quantisation the activation
quantisation kernels use (quantize_one_r in ternary_matvec_amd/csrc/actq.hpp).

The per-token code is clip(rint(v / s), -128, 127) with v / s an IEEE fp32
division (the quantisation formula of the cpp20gemma README and the ternary
page's "Step 2").  The kernels instead form y = v * r with r = 1 / s, both
IEEE fp32, take rint(y) unless y lies within a threshold of a half-integer,
and divide only there.  The claim is that this gives the divided code for
every v with |v| <= m, s = max(m, 1e-9) / 127.  numpy's float32 arithmetic is
IEEE with round-to-nearest-even, as the GPU's is with the library's flags, so
both forms are evaluated here exactly as the GPU evaluates them; the threshold
is read from the source, so a change there is checked here.
"""
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "ternary_matvec_amd", "csrc", "actq.hpp")

f32 = np.float32


def _threshold():
    src = open(SRC).read()
    body = src[src.index("quantize_one_r(float v"):]
    m = re.search(r"fabsf\(y - n\) < 0\.5f - 0x1p-(\d+)f", body)
    assert m, "quantize_one_r's half-integer test not found in actq.hpp"
    return f32(0.5) - f32(2.0 ** -int(m.group(1)))


def divided(v, s):
    q = np.rint(v / s)
    return np.clip(q, -128, 127).astype(np.int8)


def multiplied(v, s, thr, count=None):
    r = f32(1.0) / s
    y = (v * r).astype(np.float32)
    n = np.rint(y)
    fast = np.abs((y - n).astype(np.float32)) < thr
    q = np.where(fast, n, np.rint(v / s))
    if count is not None:
        count.append(int((~fast).sum()))
    return np.clip(q, -128, 127).astype(np.int8)


def _scale(m):
    return (np.maximum(f32(m), f32(1e-9)) / f32(127.0)).astype(np.float32)


def _rows(rng, n, k, std):
    return (rng.standard_normal((n, k)) * std).astype(np.float32)


def test_random_rows_equal_division():
    thr = _threshold()
    rng = np.random.default_rng(20261202)
    slow = []
    for std in (1e-8, 1e-3, 0.02, 1.0, 3.7, 1e3, 1e12):
        x = _rows(rng, 64, 4096, std)
        m = np.abs(x).max(axis=1, keepdims=True)
        s = _scale(m)
        np.testing.assert_array_equal(multiplied(x, s, thr, slow), divided(x, s))
    # the division is the exception: a few per 10^4 values
    assert sum(slow) < 1e-3 * 7 * 64 * 4096


def test_exact_half_integers_round_to_even():
    """v / s exactly j + 1/2 (s a power of two): the multiply can land on
    either side; the code must be the division's half-to-even rounding."""
    thr = _threshold()
    for e in range(-20, 21, 3):
        s = f32(2.0 ** e)
        j = np.arange(-127, 127, dtype=np.float32)
        v = ((j + f32(0.5)) * s).astype(np.float32)
        got = multiplied(v, np.full_like(v, s), thr)
        np.testing.assert_array_equal(got, divided(v, np.full_like(v, s)))
        assert got[127] == 0 and got[128] == 2 and got[126] == 0   # 0.5 -> 0, 1.5 -> 2, -0.5 -> -0


def test_values_next_to_half_integers():
    """v within a few ulps of (j + 1/2) s for scales with full mantissas: the
    cases where v * r and v / s round to different floats."""
    thr = _threshold()
    rng = np.random.default_rng(7)
    s = _scale((rng.uniform(0.5, 2.0, 2000) * 127).astype(np.float32) * f32(0.37))
    j = rng.integers(-127, 127, 2000).astype(np.float32)
    base = ((j + f32(0.5)) * s).astype(np.float32)
    for steps in range(-4, 5):
        v = base.copy()
        for _ in range(abs(steps)):
            v = np.nextafter(v, np.float32(np.inf if steps > 0 else -np.inf)).astype(np.float32)
        np.testing.assert_array_equal(multiplied(v, s, thr), divided(v, s))


def test_a_zero_threshold_would_be_wrong():
    """The threshold matters: deciding on y alone (no division near half-integers) gives other codes."""
    rng = np.random.default_rng(11)
    s = _scale((rng.uniform(0.5, 2.0, 20000) * 127).astype(np.float32) * f32(0.37))
    j = rng.integers(-127, 127, 20000).astype(np.float32)
    v = ((j + f32(0.5)) * s).astype(np.float32)
    naive = np.clip(np.rint((v * (f32(1.0) / s)).astype(np.float32)), -128, 127).astype(np.int8)
    assert (naive != divided(v, s)).any()
    np.testing.assert_array_equal(multiplied(v, s, _threshold()), divided(v, s))


def test_row_extremes_and_zero_rows():
    thr = _threshold()
    x = np.zeros((3, 100), dtype=np.float32)
    x[1, 5] = f32(-3.0e38)
    x[1, 6] = f32(1e-40)                      # subnormal
    x[2, :] = -0.0
    m = np.abs(x).max(axis=1, keepdims=True)
    s = _scale(m)
    np.testing.assert_array_equal(multiplied(x, s, thr), divided(x, s))
    assert multiplied(x, s, thr)[1, 5] == -127
