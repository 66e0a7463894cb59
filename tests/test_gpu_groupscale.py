"""GPU parity of the group-scaled int8 path (weights in groups of 128 columns,
activations in groups of 32) against the CPU oracle, through the C ABI.

  * qmv_quantize_act_grouped and qmv_pack_int8_grouped: codes, padding bytes
    and scales bit-exact;
  * qmv_gemv on QMV_W_INT8_G128 problems: every output within
    (ceil(k/32) + 3) * 2^-24 * sum_h |term_h| of the oracle's fp64 value (the
    GPU forms each term with one fp32 product and one fused multiply-add and
    sums the terms in fp32; the oracle returns sum_h |term_h|);
  * the same problems mixed with ternary and per-tensor int8 ones in one call.
Shapes: ragged k (1, 17, 70, 300), every lanes-per-row choice (4 .. 64), rows
not a multiple of a tile, 1 to 16 tokens, the Gemma-3-1B layer shapes.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from ternary_matvec_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _stride(k):
    return (k + 15) // 16 * 16


@pytest.mark.parametrize("m,k", [(1, 1), (1, 31), (2, 33), (3, 70), (1, 1152), (16, 6912), (5, 300), (2, 4097)])
def test_quantize_act_grouped_bit_exact(qmv_gpu, m, k):
    from ternary_matvec_amd import qmv
    say("quantize_act_grouped", m, k)
    x = synth.normal(11000 + k + m, (m, k), std=2.0)
    if m > 1:
        x[1, :] = 0.0                              # zero row: floor scales, zero codes
    if k >= 40:
        x[0, 32:40] = [0.5, -0.5, 2.5, -2.5, 1.5, 127.0, -127.0, 0.0]   # exact halves in one group
    q_ref, s_ref = oracle.quantize_groups(x, 32)
    x8, sx = qmv.qmv_quantize_act_grouped(_t(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(x8.cpu().numpy(), q_ref)


@pytest.mark.parametrize("n,k", [(768, 288), (3, 300), (1152, 6912), (5, 1), (7, 129), (64, 17)])
def test_pack_int8_grouped_bit_exact(qmv_gpu, n, k):
    from ternary_matvec_amd import qmv
    say("pack_int8_grouped", n, k)
    w = synth.normal(12000 + k + n, (n, k), std=0.02)
    w[0, :min(k, 128)] *= 50.0                     # one group far larger than the rest
    q_ref, s_ref = oracle.quantize_groups(w, 128)
    packed = torch.full((qmv.qmv_packed_bytes(qmv.QMV_W_INT8_G128, n, k),), 0x5A, dtype=torch.uint8, device=DEV)
    pw = qmv.qmv_pack_int8_grouped(_t(w), packed=packed)
    torch.cuda.synchronize()
    assert pw.wtype == qmv.QMV_W_INT8_G128 and pw.scale.shape == s_ref.shape
    np.testing.assert_array_equal(pw.scale.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    got = pw.packed.cpu().numpy().view(np.int8).reshape(n, _stride(k))
    np.testing.assert_array_equal(got[:, :k], q_ref)
    assert (got[:, k:] == 0).all()                 # row padding is zero


def _case(n, k, m, seed):
    w = synth.normal(seed, (n, k), std=0.02)
    for g in range(0, k, 128):                     # distinct group magnitudes
        w[:, g:g + 128] *= np.float32(1.0 + (g // 128) % 5)
    x = synth.normal(seed + 1, (m, k))
    x[:, :min(k, 32)] *= 20.0                      # a few large dimensions
    return w, x


def _check(y, w8, sw, x8, sx):
    y_ref, bound = oracle.gemv_grouped(w8, sw, x8, sx)
    hn = (w8.shape[1] + 31) // 32
    tol = (hn + 3) * 2.0 ** -24 * bound + 1e-30
    err = np.abs(y.astype(np.float64) - y_ref)
    assert np.all(err <= tol), (float((err / np.maximum(tol, 1e-300)).max()), np.unravel_index(np.argmax(err - tol), err.shape))


GROUPED_CASES = [(1, 1, 1), (5, 17, 1), (64, 70, 3), (100, 300, 2), (768, 288, 1), (6912, 1152, 1),
                 (1152, 6912, 1), (1152, 6912, 4), (257, 1024, 16), (33, 4097, 5), (70, 2000, 8), (1000, 128, 2),
                 (3, 3000, 16)]


@pytest.mark.parametrize("n,k,m", GROUPED_CASES)
def test_gemv_groupscale_parity(qmv_gpu, n, k, m):
    from ternary_matvec_amd import qmv
    say("gemv group-scaled", n, k, m)
    w, x = _case(n, k, m, 13000 + n + k + m)
    pw = qmv.qmv_pack_int8_grouped(_t(w))
    x8, sx = qmv.qmv_quantize_act_grouped(_t(x))
    p = qmv.Problem(pw, x8, sx)
    p.y.fill_(float("nan"))
    qmv.qmv_gemv([p])
    torch.cuda.synchronize()
    w8, sw = oracle.quantize_groups(w, 128)
    q, s = oracle.quantize_groups(x, 32)
    _check(p.y.cpu().numpy(), w8, sw, q, s)


def test_gemv_groupscale_mixed_with_other_types_and_repeated(qmv_gpu):
    from ternary_matvec_amd import qmv
    say("gemv group-scaled mixed with ternary and int8, two calls on one workspace")
    probs, checks = [], []
    for i, (n, k, m) in enumerate([(300, 1152, 1), (64, 6912, 2), (1024, 1152, 1)]):
        w, x = _case(n, k, m, 14000 + 10 * i)
        pw = qmv.qmv_pack_int8_grouped(_t(w))
        x8, sx = qmv.qmv_quantize_act_grouped(_t(x))
        probs.append(qmv.Problem(pw, x8, sx))
        checks.append(("g", w, x))
    t = synth.trits(14100, (500, 1152))
    xt = synth.normal(14101, (1, 1152))
    qt, st = oracle.quantize_rows(xt)
    probs.append(qmv.Problem(qmv.qmv_pack_ternary(_t(t), 0.5), _t(qt), _t(st),
                             acc=torch.zeros((1, 500), dtype=torch.int32, device=DEV)))
    checks.append(("t", t, qt))
    wi = synth.normal(14102, (200, 288), std=0.02)
    qwi, swi = oracle.quantize_tensor(wi)
    xi = synth.normal(14103, (2, 288))
    qi, si = oracle.quantize_rows(xi)
    probs.append(qmv.Problem(qmv.qmv_pack_int8(_t(wi)), _t(qi), _t(si),
                             acc=torch.zeros((2, 200), dtype=torch.int32, device=DEV)))
    checks.append(("i", qwi, qi))
    plan = qmv.gemv_plan(probs)
    plan.launch()
    torch.cuda.synchronize()
    first = [p.y.clone() for p in probs]
    for p in probs:
        p.y.zero_()
    plan.launch()
    torch.cuda.synchronize()
    for p, f in zip(probs, first):
        assert torch.equal(p.y, f)
    for p, c in zip(probs, checks):
        if c[0] == "g":
            w8, sw = oracle.quantize_groups(c[1], 128)
            q, s = oracle.quantize_groups(c[2], 32)
            _check(p.y.cpu().numpy(), w8, sw, q, s)
        else:
            np.testing.assert_array_equal(p.acc.cpu().numpy(), oracle.matmul_int(c[2], c[1]))


def test_gemv_groupscale_gemma_layer(qmv_gpu):
    from ternary_matvec_amd import qmv
    say("gemv group-scaled: one Gemma-3-1B layer (6 matrices) in one call, 1 token")
    probs, refs = [], []
    for i, (name, n, k) in enumerate(synth.GEMMA_MATS):
        w, x = _case(n, k, 1, 15000 + 10 * i)
        pw = qmv.qmv_pack_int8_grouped(_t(w))
        x8, sx = qmv.qmv_quantize_act_grouped(_t(x))
        probs.append(qmv.Problem(pw, x8, sx))
        refs.append((w, x))
    qmv.qmv_gemv(probs)
    torch.cuda.synchronize()
    for p, (w, x) in zip(probs, refs):
        w8, sw = oracle.quantize_groups(w, 128)
        q, s = oracle.quantize_groups(x, 32)
        _check(p.y.cpu().numpy(), w8, sw, q, s)
