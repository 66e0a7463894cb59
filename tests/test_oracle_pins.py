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
# O7 sketch head
# --------------------------------------------------------------------------

def _bf16(a):
    return synth.to_bf16_bits(np.asarray(a, np.float32))


def test_sketch_signs_closed_form():
    # row 0 all negative, row 1 negative at even columns, row 2 all positive; k = 40 spans two words
    k = 40
    w = np.stack([np.full(k, -0.5), np.where(np.arange(k) % 2 == 0, -0.5, 0.5), np.full(k, 0.25)])
    bits = oracle.sketch_signs(_bf16(w))
    assert bits.shape == (2, 3)
    np.testing.assert_array_equal(bits[:, 0], [0xFFFFFFFF, 0xFF])
    np.testing.assert_array_equal(bits[:, 1], [0x55555555, 0x55])
    np.testing.assert_array_equal(bits[:, 2], [0, 0])
    # zero and negative zero count as positive
    z = _bf16(np.array([[0.0, -0.0, -1.0]], np.float32))
    np.testing.assert_array_equal(oracle.sketch_signs(z)[:, 0], [0b100])


def test_sketch_scale_closed_form():
    w = _bf16(np.where(np.arange(600 * 40).reshape(600, 40) % 3 == 0, -0.25, 0.25))
    assert oracle.sketch_scale(w) == np.float32(0.25)
    w2 = _bf16(np.concatenate([np.full((300, 8), 0.5), np.full((300, 8), -1.5)]))
    assert oracle.sketch_scale(w2) == np.float32(1.0)


@pytest.mark.parametrize("k,sizes", [(1152, [280, 280, 280, 280]), (37, [1, 1, 1, 2]), (33, [0, 0, 0, 1]),
                                     (20, [0, 0, 0, 0]), (100, [17, 17, 17, 17])])
def test_sketch_plan_group_sizes(k, sizes):
    x = synth.normal(41, (k,))
    top_idx, group_of, group_n, group_w = oracle.sketch_plan(x, 1.0)
    t = min(32, k)
    assert len(top_idx) == t
    assert list(group_n) == sizes
    assert sorted(set(top_idx.tolist())) == sorted(top_idx.tolist())          # distinct
    assert np.all(group_of[top_idx] == -1)
    for g in range(4):
        assert int((group_of == g).sum()) == sizes[g]
    # the exact dimensions are the t largest |x|, in descending order
    mags = np.abs(x)
    assert np.all(np.diff(mags[top_idx]) <= 0)
    rest = np.setdiff1d(np.arange(k), top_idx)
    if rest.size:
        assert mags[rest].max() <= mags[top_idx].min()
    # groups follow the rank order: every |x| of group g is >= every |x| of group g + 1
    for g in range(3):
        if sizes[g] and sizes[g + 1]:
            assert mags[group_of == g].min() >= mags[group_of == g + 1].max()


def test_sketch_plan_ties_and_group_weights_closed_form():
    # |x| = k - i: ranks are the indices in order; ties (all equal) also rank by index
    k = 72
    x = np.array([(k - i) * (-1) ** i for i in range(k)], np.float32)
    top_idx, group_of, group_n, group_w = oracle.sketch_plan(x, 0.5)
    np.testing.assert_array_equal(top_idx, np.arange(32))
    assert list(group_n) == [10, 10, 10, 10]
    # group g holds ranks 32+10g .. 41+10g, |x| = 40-10g .. 31-10g: mean = 35.5 - 10 g
    np.testing.assert_array_equal(group_w, 0.5 * np.array([35.5, 25.5, 15.5, 5.5]))
    eq = np.ones(50, np.float32)
    top_idx, _, _, _ = oracle.sketch_plan(eq, 1.0)
    np.testing.assert_array_equal(top_idx, np.arange(32))


def test_sketch_scores_equal_exact_logits_when_all_magnitudes_match():
    # |w| = 0.5 and |x| = 1 everywhere: c = 0.5, every group weight is 0.5 and every
    # product w*x = 0.5 * (sign agreement), so steps 1 + 2 reproduce the exact logit
    # exactly (small multiples of 0.5); a dropped, doubled or mis-signed dimension breaks it
    v, k = 300, 200
    sw = np.where(synth.raw(43, v * k).reshape(v, k) % 2 == 0, 1.0, -1.0)
    sx = np.where(synth.raw(44, k) % 2 == 0, 1.0, -1.0).astype(np.float32)
    w = _bf16(0.5 * sw)
    assert oracle.sketch_scale(w) == 0.5
    scores, mag = oracle.sketch_scores(w, sx, 0.5)
    exact = (0.5 * sw) @ sx
    np.testing.assert_array_equal(scores, exact)
    # the magnitude is 0.5 per exact dimension plus 0.5 |agreement| per group
    assert np.all(mag >= np.abs(scores)) and np.all(mag <= 0.5 * k)
    assert np.all(mag >= 0.5 * 32)


def test_sketch_scores_brute_force_tiny():
    # v = 3, k = 36 by hand: 32 exact dimensions, then groups of 1, 1, 1, 1 (k - T = 4)
    k = 36
    x = np.array([36 - i for i in range(k)], np.float32)          # ranks = indices
    w = np.zeros((3, k), np.float32)
    w[0, :] = 0.25                                                  # all signs agree
    w[1, :] = -0.25                                                 # all disagree
    w[2, :32] = 0.0
    w[2, 32:] = [0.5, -0.5, 0.5, -0.5]
    wb = _bf16(w)
    c = oracle.sketch_scale(wb)
    assert c == (0.25 * 36 * 2 + 0.5 * 4) / (3 * 36)
    scores, _ = oracle.sketch_scores(wb, x, c)
    exact32 = 0.25 * sum(36 - i for i in range(32))
    tail = c * np.array([4.0, 3.0, 2.0, 1.0])                       # group weights c * |x| of ranks 32..35
    np.testing.assert_allclose(scores, [exact32 + tail.sum(), -exact32 - tail.sum(),
                                        tail[0] - tail[1] + tail[2] - tail[3]], rtol=1e-15)


def test_sketch_scores_sign_symmetry():
    v, k = 64, 1152
    w = _bf16(synth.normal(45, (v, k), std=0.02))
    x = synth.normal(46, (k,))
    c = oracle.sketch_scale(w)
    s1, m1 = oracle.sketch_scores(w, x, c)
    s2, m2 = oracle.sketch_scores(w ^ np.uint16(0x8000), x, c)    # every weight negated
    zero = (w & np.uint16(0x7FFF)) == 0
    assert not zero.any()
    np.testing.assert_array_equal(s2, -s1)
    np.testing.assert_array_equal(m2, m1)


def test_sketch_pick_all_exact_matches_full_argmax():
    # k <= 32: every dimension is exact, so the best word always makes the candidates
    for seed in range(5):
        w = _bf16(synth.normal(50 + seed, (3000, 32), std=0.02))
        x = synth.normal(60 + seed, (32,))
        idx, cand, scores, logits = oracle.sketch_head(w, x)
        full, fidx = oracle.lmhead(w, x)
        assert idx == fidx
        assert cand.sum() == 1024
        np.testing.assert_array_equal(logits[cand], full[cand])


def test_sketch_pick_candidates_are_the_best_scores():
    v, k = 5000, 256
    w = _bf16(synth.normal(47, (v, k), std=0.02))
    x = synth.normal(48, (k,))
    idx, cand, scores, logits = oracle.sketch_head(w, x)
    assert cand.sum() == 1024
    assert scores[cand].min() >= scores[~cand].max()
    assert idx == int(np.flatnonzero(cand)[np.argmax(logits[cand].astype(np.float32))])
    # fewer words than 1024: every word is a candidate and the pick is the full argmax
    idx2, cand2, _, _ = oracle.sketch_head(w[:700], x)
    assert cand2.all() and idx2 == oracle.lmhead(w[:700], x)[1]


def test_sketch_pick_ties_at_the_cut_go_to_the_lower_index():
    # 150 of the 1200 words are copies of the word ranked about 1000th, so the 1024th
    # best score is tied: exactly the copies with the lowest indices make the cut
    v, k = 1200, 64
    w = _bf16(synth.normal(52, (v, k), std=0.02))
    x = synth.normal(53, (k,))
    s, _ = oracle.sketch_scores(w, x, oracle.sketch_scale(w))
    order = np.argsort(-s, kind="stable")
    template = order[990]
    w[order[1040:1190]] = w[template]
    s, _ = oracle.sketch_scores(w, x, oracle.sketch_scale(w))
    ties = np.flatnonzero(s == s[template])
    above = int((s > s[template]).sum())
    assert ties.size == 151 and above < 1024 < above + ties.size
    cand, _, _ = oracle.sketch_pick(w, x, s)
    assert cand.sum() == 1024
    np.testing.assert_array_equal(np.flatnonzero(cand & (s == s[template])), ties[:1024 - above])
    assert np.all(cand[s > s[template]]) and not np.any(cand[s < s[template]])


def test_sketch_pick_planted_winner():
    v, k = 20000, 1152
    w = _bf16(synth.normal(49, (v, k), std=0.02))
    wf = synth.bf16_bits_to_f32(w)
    x = (40.0 * wf[12345] + synth.normal(51, (k,)) * 0.2).astype(np.float32)
    idx, cand, _, _ = oracle.sketch_head(w, x)
    assert cand[12345] and idx == 12345 == oracle.lmhead(w, x)[1]


# --------------------------------------------------------------------------
# O8 fused RMSNorm / gated activation before quantisation
# --------------------------------------------------------------------------

def test_rmsnorm_matches_definition_and_is_scale_invariant():
    import math
    for m, k in [(3, 1152), (2, 257), (1, 1), (4, 6912)]:
        x = synth.normal(81 + k, (m, k))
        w = synth.normal(82 + k, (k,)) * 0.5 + 1.0
        o = oracle.rmsnorm(x, w, 1e-5)
        # the definition in exact rationals, then one square root: within a few fp64 roundings
        for r in range(m):
            ss = sum(Fraction(float(v)) ** 2 for v in x[r])
            ms = ss / k + Fraction(1e-5)
            for j in (0, k // 2, k - 1):
                ref = Fraction(float(w[j])) * Fraction(float(x[r, j]))
                # o^2 * ms = ref^2 up to the roundings of sqrt and the divide
                lhs = Fraction(float(o[r, j])) ** 2 * ms
                assert abs(lhs - ref ** 2) <= Fraction(1, 10 ** 13) * ref ** 2 + Fraction(1, 10 ** 300)
            np.testing.assert_allclose(o[r], w.astype(np.float64) * x[r].astype(np.float64) /
                                       math.sqrt(float(ss / k) + 1e-5), rtol=1e-14, atol=0)
        # eps = 0: scaling x by a power of two changes nothing, bit for bit
        o0 = oracle.rmsnorm(x, w, 0.0)
        o1 = oracle.rmsnorm(x * np.float32(8.0), w, 0.0)
        np.testing.assert_array_equal(o0, o1)
    # unit weights: the output's mean square is 1 / (1 + eps / mean(x^2))
    x = synth.normal(85, (1, 4096))
    o = oracle.rmsnorm(x, np.ones(4096, np.float32), 1e-5)
    ms = float(np.mean(x.astype(np.float64) ** 2))
    assert abs(float(np.mean(o ** 2)) - 1.0 / (1.0 + 1e-5 / ms)) < 1e-12
    # a constant row of c with eps = 0 normalises to exactly +-1
    o = oracle.rmsnorm(np.full((1, 10), -3.0, np.float32), np.ones(10, np.float32), 0.0)
    np.testing.assert_array_equal(o, -np.ones((1, 10)))


def test_glu_matches_library_activations():
    import torch
    g = np.concatenate([synth.normal(86, (1, 500)) * 4.0, np.array([[0.0, -0.0, 30.0, -30.0, 1.0]], np.float32)], 1)
    u = synth.normal(87, g.shape)
    gt = torch.from_numpy(g.astype(np.float64))
    ut = torch.from_numpy(u.astype(np.float64))
    ref_gelu = (torch.nn.functional.gelu(gt, approximate="tanh") * ut).numpy()
    ref_silu = (torch.nn.functional.silu(gt) * ut).numpy()
    np.testing.assert_allclose(oracle.glu(g, u, oracle.GLU_GELU_TANH), ref_gelu, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.glu(g, u, oracle.GLU_SILU), ref_silu, rtol=1e-13, atol=1e-15)
    h = oracle.glu(np.zeros((1, 4), np.float32), np.ones((1, 4), np.float32), oracle.GLU_GELU_TANH)
    assert np.all(h == 0.0)


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


# --------------------------------------------------------------------------
# O9 group-wise scales (the gemma.cpp tour, "Weights, Blobs, and the .sbs
# Format": int8 groups of 128 sharing a scale; [T] "A side finding: Gemma 4
# E4B in 4-bit": one activation scale per 32 values).
# --------------------------------------------------------------------------

@pytest.mark.parametrize("k", [1, 31, 32, 33, 128, 300, 1152])
def test_groups_of_a_whole_row_are_per_row_quantisation(k):
    x = synth.normal(91 + k, (3, k))
    q1, s1 = oracle.quantize_rows(x)
    for g in (k, k + 1, 4 * k):
        q, s = oracle.quantize_groups(x, g)
        assert s.shape == (3, 1)
        np.testing.assert_array_equal(q, q1)
        np.testing.assert_array_equal(s[:, 0].view(np.uint32), s1.view(np.uint32))


def test_groups_closed_form_and_ragged_tail():
    # k = 70 in groups of 32: [0, 32), [32, 64), [64, 70)
    x = np.zeros((1, 70), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 2.0, -2.0, 1.0          # group 0: absmax 2 -> codes 127, -127, 64 (63.5 -> 64)
    x[0, 40] = -0.5                                      # group 1: absmax 0.5 -> -127
    x[0, 69] = 3.0                                       # tail group of 6 columns
    q, s = oracle.quantize_groups(x, 32)
    assert s.shape == (1, 3)
    assert s[0].tolist() == [np.float32(2.0) / np.float32(127.0), np.float32(0.5) / np.float32(127.0),
                             np.float32(3.0) / np.float32(127.0)]
    assert (q[0, :3] == [127, -127, 64]).all() and (q[0, 3:32] == 0).all()
    assert q[0, 40] == -127 and q[0, 69] == 127
    # an all-zero group takes the floor scale and zero codes
    q0, s0 = oracle.quantize_groups(np.zeros((2, 64), np.float32), 32)
    assert (q0 == 0).all() and (s0 == np.float32(1e-9) / np.float32(127.0)).all()


def test_groups_are_independent_of_each_other_and_of_other_rows():
    x = synth.normal(93, (2, 300))
    q, s = oracle.quantize_groups(x, 128)
    y = x.copy()
    y[0, 130] = 1000.0            # only row 0, group 1 may change
    q2, s2 = oracle.quantize_groups(y, 128)
    changed = (q2 != q)
    assert not changed[1].any() and not changed[0, :128].any() and not changed[0, 256:].any()
    assert changed[0, 128:256].any()
    assert (s2 != s).sum() == 1 and s2[0, 1] != s[0, 1]
    # each group's codes equal per-row quantisation of that group alone
    for g, (c0, c1) in enumerate([(0, 128), (128, 256), (256, 300)]):
        qg, sg = oracle.quantize_rows(x[:, c0:c1])
        np.testing.assert_array_equal(q[:, c0:c1], qg)
        np.testing.assert_array_equal(s[:, g], sg)


def _equal_absmax(seed, shape, group, amax):
    """Values in [-amax/2, amax/2] with +-amax planted once in every group."""
    m, k = shape
    v = ((synth.uniform(seed, m * k).reshape(m, k) - 0.5) * amax).astype(np.float32)
    for c0 in range(0, k, group):
        v[:, c0] = amax if (c0 // group) % 2 == 0 else -amax
    return v


@pytest.mark.parametrize("m,n,k", [(1, 5, 256), (3, 7, 300), (2, 4, 1152)])
def test_gemv_grouped_with_equal_scales_is_the_exact_int_path(m, n, k):
    # every weight group and every activation group has the same absmax, so all
    # scales are equal and y must be the per-tensor result acc * sx * sw
    w = _equal_absmax(94 + k, (n, k), 128, 0.75)
    x = _equal_absmax(95 + k, (m, k), 32, 3.0)
    w8, sw = oracle.quantize_groups(w, 128)
    x8, sx = oracle.quantize_groups(x, 32)
    assert len(set(sw.ravel().tolist())) == 1 and len(set(sx.ravel().tolist())) == 1
    y, bound = oracle.gemv_grouped(w8, sw, x8, sx)
    acc = oracle.matmul_int(x8, w8)
    ref = acc.astype(np.float64) * float(sx[0, 0]) * float(sw[0, 0])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-300)
    assert (bound >= np.abs(y) * (1 - 1e-12)).all()


def test_gemv_grouped_maps_activation_group_h_to_weight_group_h_div_4():
    # x is zero outside activation group h0; weight groups have distinct scales
    n, k = 6, 640                       # 5 weight groups, 20 activation groups
    w = synth.normal(96, (n, k))
    for g in range(5):
        w[:, 128 * g:128 * g + 128] *= np.float32(1 + 3 * g)
    w8, sw = oracle.quantize_groups(w, 128)
    for h0 in (0, 3, 4, 5, 19):
        x = np.zeros((1, k), np.float32)
        x[0, 32 * h0:32 * h0 + 32] = synth.normal(97 + h0, (32,))
        x8, sx = oracle.quantize_groups(x, 32)
        y, _ = oracle.gemv_grouped(w8, sw, x8, sx)
        d = oracle.matmul_int(x8[:, 32 * h0:32 * h0 + 32], w8[:, 32 * h0:32 * h0 + 32])
        ref = d[0].astype(np.float64) * sw[:, h0 // 4].astype(np.float64) * float(sx[0, h0])
        np.testing.assert_allclose(y[0], ref, rtol=1e-13, atol=0)


def test_gemv_grouped_tiny_exact_rationals():
    m, n, k = 2, 3, 70
    w8, sw = oracle.quantize_groups(synth.normal(98, (n, k)), 128)
    x8, sx = oracle.quantize_groups(synth.normal(99, (m, k)), 32)
    y, _ = oracle.gemv_grouped(w8, sw, x8, sx)
    for mi, r in itertools.product(range(m), range(n)):
        exact = sum(Fraction(float(sw[r, c // 128])) * Fraction(float(sx[mi, c // 32])) * int(x8[mi, c]) * int(w8[r, c])
                    for c in range(k))
        assert abs(Fraction(y[mi, r]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 1000)
