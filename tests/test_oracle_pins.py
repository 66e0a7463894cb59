"""Pins of the CPU oracle to what the pages and mathematics fix (CPU only).

Every test here checks the oracle against something other than itself:
values derived by hand from the pages' definitions (tests/golden), closed
forms, exact rational arithmetic, exhaustive enumeration and brute force with
Python integers on tiny inputs.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from ternary_matvec_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _nearest_f32(fr: Fraction) -> np.float32:
    """The fp32 value nearest to an exact rational (ties to even mantissa)."""
    f = np.float32(float(fr))  # within one ulp
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        if best is None or d < best[0] or (d == best[0] and int(cand.view(np.uint32)) % 2 == 0):
            best = (d, cand)
    return best[1]


# --------------------------------------------------------------------------
# O1 quantisation
# --------------------------------------------------------------------------

def test_quantize_half_even_golden():
    rows = _read_golden("quantize_half_even.txt")
    x = np.array([float(r[0]) for r in rows], np.float32)
    want = np.array([int(r[1]) for r in rows], np.int8)
    q, s = oracle.quantize_rows(x[None, :])
    assert s[0] == np.float32(1.0)
    np.testing.assert_array_equal(q[0], want)


def test_quantize_zero_row_uses_floor():
    q, s = oracle.quantize_rows(np.zeros((1, 33), np.float32))
    assert np.all(q == 0)
    assert s[0] == _nearest_f32(Fraction(float(np.float32(1e-9))) / 127)


def test_quantize_scale_is_correctly_rounded_max_over_127():
    x = synth.normal(11, (64, 300))
    x[5, 17] = -9.75  # an exact negative maximum
    q, s = oracle.quantize_rows(x)
    for r in range(x.shape[0]):
        m = max(abs(Fraction(float(v))) for v in x[r])
        assert s[r] == _nearest_f32(m / 127), r


def test_quantize_invariants_exact():
    x = synth.normal(12, (32, 257), std=3.0)
    q, s = oracle.quantize_rows(x)
    assert q.min() >= -127 and q.max() <= 127
    for r in range(x.shape[0]):
        a = int(np.argmax(np.abs(x[r])))
        assert abs(int(q[r, a])) == 127
        assert np.sign(q[r, a]) == np.sign(x[r, a])
        sr = Fraction(float(s[r]))
        for c in range(0, x.shape[1], 7):
            exact = Fraction(float(x[r, c])) / sr
            # rounding of the fp32 quotient adds at most half an ulp of a value below 128
            assert abs(exact - int(q[r, c])) <= Fraction(1, 2) + Fraction(1, 1 << 17)


def test_quantize_tensor_has_one_scale():
    w = synth.normal(13, (48, 40), std=0.02)
    w[31, 3] = 0.5
    q, s = oracle.quantize_tensor(w)
    assert s == _nearest_f32(Fraction(0.5) / 127)
    assert q[31, 3] == 127
    # a row with small values keeps the tensor scale, so its codes are small
    assert np.abs(q[0]).max() < 20


def test_quantize_dequant_error_bound():
    # cpp20gemma: dequantised weights are w8 * scale; the error is at most half a step
    w = synth.normal(14, (20, 64), std=0.02)
    q, s = oracle.quantize_tensor(w)
    err = np.abs(q.astype(np.float64) * float(s) - w.astype(np.float64))
    assert err.max() <= 0.5 * float(s) * (1 + 1e-6)


# --------------------------------------------------------------------------
# O2 trit5 packing
# --------------------------------------------------------------------------

def test_pack_all_243_codes():
    tuples = list(itertools.product((-1, 0, 1), repeat=5))
    t = np.array(tuples, np.int8)                     # 243 rows x 5 columns
    packed, bad = oracle.pack_trit5(t)
    assert bad == 0
    n = len(tuples)
    codes = []
    for r, tup in enumerate(tuples):
        # base 3, column 5j+i is digit i; write the digits most significant first
        want = int("".join(str(v + 1) for v in reversed(tup)), 3)
        got = int(packed[r * 16 + 0])                 # chunk 0 of row r
        assert got == want, (tup, got, want)
        codes.append(got)
        # the other 15 bytes of the row are padding
        assert np.all(packed[r * 16 + 1: r * 16 + 16] == 121)
    assert sorted(codes) == list(range(243))
    back, invalid = oracle.unpack_trit5(packed, n, 5)
    assert invalid == 0
    np.testing.assert_array_equal(back, t)


def test_pack_layout_golden_3x81():
    rows = _read_golden("trit5_layout_3x81.txt")
    want = np.array([int(v) for r in rows for v in r], np.uint8)
    t = np.stack([np.full(81, 1), np.zeros(81), np.full(81, -1)]).astype(np.int8)
    packed, bad = oracle.pack_trit5(t)
    assert bad == 0
    np.testing.assert_array_equal(packed, want)


@pytest.mark.parametrize("k", [1, 4, 5, 6, 7, 23, 79, 80, 81, 288, 1152])
def test_pack_sizes_roundtrip(k):
    n = 9
    t = synth.trits(100 + k, (n, k))
    packed, bad = oracle.pack_trit5(t)
    stride = -(-(-(-k // 5)) // 16) * 16
    assert oracle.trit5_row_bytes(k) == -(-k // 5)
    assert oracle.trit5_row_stride(k) == stride
    assert packed.size == n * stride and bad == 0
    assert packed.max() < 243
    back, invalid = oracle.unpack_trit5(packed, n, k)
    assert invalid == 0
    np.testing.assert_array_equal(back, t)


def test_pack_counts_bad_trits_and_packs_them_as_zero():
    t = np.array([[1, 2, -1, -3, 0, 5, 0]], np.int8)
    packed, bad = oracle.pack_trit5(t)
    assert bad == 3
    back, _ = oracle.unpack_trit5(packed, 1, 7)
    np.testing.assert_array_equal(back, [[1, 0, -1, 0, 0, 0, 0]])


def test_unpack_flags_invalid_codes():
    packed = np.full(16, 121, np.uint8)
    packed[0] = 250
    t, invalid = oracle.unpack_trit5(packed, 1, 10)
    assert invalid == 1
    assert np.all(t[0, :5] == 0)


def test_int8_layout_golden():
    # 2 x 20 int8 codes: row stride 32 bytes = 2 chunks; chunk-major device order
    q = np.arange(40, dtype=np.int8).reshape(2, 20) - 20
    out = oracle.layout_int8(q)
    want = np.zeros(64, np.int8)
    want[0:16] = q[0, 0:16]
    want[16:32] = q[1, 0:16]
    want[32:36] = q[0, 16:20]
    want[48:52] = q[1, 16:20]
    np.testing.assert_array_equal(out, want)


# --------------------------------------------------------------------------
# O4 integer core
# --------------------------------------------------------------------------

def _brute_int(x8, w):
    m, k = x8.shape
    n = w.shape[0]
    out = [[0] * n for _ in range(m)]
    for a in range(m):
        for b in range(n):
            s = 0
            for c in range(k):
                s += int(x8[a, c]) * int(w[b, c])
            out[a][b] = s
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (1, 3, 4), (2, 5, 5), (3, 4, 6), (1, 16, 7), (4, 7, 23), (2, 16, 16)])
def test_matmul_bruteforce_ternary(m, n, k):
    x8 = (synth.raw(200 + k, m * k) % np.uint64(256)).astype(np.int64).astype(np.uint8).view(np.int8).reshape(m, k)
    t = synth.trits(300 + k, (n, k))
    acc = oracle.matmul_int(x8, t)
    np.testing.assert_array_equal(acc, _brute_int(x8, t))


def test_matmul_bruteforce_int8_weights():
    x8 = (synth.raw(7, 3 * 19) % np.uint64(256)).astype(np.uint8).view(np.int8).reshape(3, 19)
    w = (synth.raw(8, 5 * 19) % np.uint64(256)).astype(np.uint8).view(np.int8).reshape(5, 19)
    np.testing.assert_array_equal(oracle.matmul_int(x8, w), _brute_int(x8, w))


def test_matmul_identities():
    k = 1152
    x8 = (synth.raw(9, k) % np.uint64(255)).astype(np.int64) - 127
    x8 = x8.astype(np.int8)[None, :]
    ones = np.ones((1, k), np.int8)
    assert oracle.matmul_int(x8, ones)[0, 0] == int(x8.astype(np.int64).sum())
    assert oracle.matmul_int(x8, -ones)[0, 0] == -int(x8.astype(np.int64).sum())
    assert oracle.matmul_int(x8, np.zeros((1, k), np.int8))[0, 0] == 0
    for j in (0, 1, 4, 5, 511, 1151):
        e = np.zeros((1, k), np.int8)
        e[0, j] = 1
        assert oracle.matmul_int(x8, e)[0, 0] == int(x8[0, j])


def test_matmul_all_243_byte_patterns():
    t = np.array(list(itertools.product((-1, 0, 1), repeat=5)), np.int8)
    x8 = np.array([[-128, 127, -5, 3, 77]], np.int8)
    acc = oracle.matmul_int(x8, t)[0]
    for r, tup in enumerate(t):
        assert acc[r] == sum(int(a) * int(b) for a, b in zip(x8[0], tup))


def test_matmul_is_batch_and_thread_invariant():
    x8 = (synth.raw(10, 16 * 300) % np.uint64(256)).astype(np.uint8).view(np.int8).reshape(16, 300)
    t = synth.trits(11, (64, 300))
    full = oracle.matmul_int(x8, t, threads=4)
    for a in (0, 7, 15):
        np.testing.assert_array_equal(oracle.matmul_int(x8[a:a + 1], t, threads=1)[0], full[a])


def test_matmul_overflow_is_reported():
    k = 140000
    x8 = np.full((1, k), -128, np.int8)
    w = np.full((1, k), -128, np.int8)
    with pytest.raises(OverflowError):
        oracle.matmul_int(x8, w)


# --------------------------------------------------------------------------
# O5 dequantisation
# --------------------------------------------------------------------------

def test_dequant_is_correctly_rounded_product():
    acc = np.array([[0, 1, -1, 877824, -877824, 123457, -99991]], np.int32)
    sx = np.array([0.0123456789], np.float32)
    sw = np.float32(0.0217)
    y = oracle.dequant(acc, sx, sw)
    assert y[0, 0] == 0.0
    for j in range(acc.shape[1]):
        exact = Fraction(int(acc[0, j])) * Fraction(float(sx[0])) * Fraction(float(sw))
        # one fp64 rounding then one fp32 rounding: within half an fp32 ulp plus 2^-52 relative
        assert abs(Fraction(float(y[0, j])) - exact) <= abs(exact) * Fraction(1, 1 << 24) * Fraction(1 + 2 ** -27)


def test_dequant_after_dot_identity():
    # cpp20gemma: (x . w8) * scale equals the dot of the dequantised vectors
    x = synth.normal(21, (3, 96))
    t = synth.trits(22, (10, 96))
    sw = 0.02
    q, sx = oracle.quantize_rows(x)
    y = oracle.dequant(oracle.matmul_int(q, t), sx, sw).astype(np.float64)
    deq = (q.astype(np.float64) * sx.astype(np.float64)[:, None]) @ (t.astype(np.float64) * float(np.float32(sw))).T
    np.testing.assert_allclose(y, deq, rtol=1e-6, atol=1e-12)


# --------------------------------------------------------------------------
# O6 output layer + greedy choice
# --------------------------------------------------------------------------

def test_lmhead_exact_on_small_case():
    w = synth.to_bf16_bits(synth.normal(31, (40, 24), std=0.5))
    x = synth.normal(32, (24,))
    logits, idx = oracle.lmhead(w, x)
    wf = synth.bf16_bits_to_f32(w)
    for r in range(40):
        exact = sum(Fraction(float(wf[r, c])) * Fraction(float(x[c])) for c in range(24))
        assert abs(Fraction(logits[r]) - exact) <= abs(exact) * Fraction(24, 1 << 52) + Fraction(1, 1 << 80)
    ex32 = [np.float32(float(sum(Fraction(float(wf[r, c])) * Fraction(float(x[c])) for c in range(24))))
            for r in range(40)]
    assert idx == int(np.argmax(ex32))


def test_lmhead_planted_winner_and_first_max_tie():
    v, k = 1000, 64
    w = synth.to_bf16_bits(synth.normal(33, (v, k), std=0.02))
    x = synth.normal(34, (k,))
    w[617] = synth.to_bf16_bits(np.sign(x) * 1.0)     # clearly dominant row
    _, idx = oracle.lmhead(w, x)
    assert idx == 617
    w[203] = w[617]                                   # exact tie: the lower index wins
    _, idx = oracle.lmhead(w, x)
    assert idx == 203


def test_lmhead_one_hot_rows_read_x():
    k = 16
    w = np.zeros((k, k), np.uint16)
    for r in range(k):
        w[r, r] = synth.to_bf16_bits(np.array([1.0], np.float32))[0]
    x = synth.normal(35, (k,))
    logits, idx = oracle.lmhead(w, x)
    np.testing.assert_array_equal(logits, x.astype(np.float64))
    assert idx == int(np.argmax(x))


# --------------------------------------------------------------------------
# The seeded generator itself (not the oracle): published splitmix64 values.
# --------------------------------------------------------------------------

def test_splitmix64_known_first_output():
    # splitmix64 with seed 0: first output 0xE220A8397B1DCDAF (reference value of the generator)
    assert int(synth.raw(0, 1)[0]) == 0xE220A8397B1DCDAF
    assert synth.splitmix64_scalar(0) == 0xE220A8397B1DCDAF


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.0], np.float32)
    b = synth.to_bf16_bits(x)
    np.testing.assert_array_equal(b, [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC000])
