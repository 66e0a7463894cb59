"""GPU parity of the fused steps either side of a GEMV (qmv_rmsnorm_quantize,
qmv_glu_quantize) against the CPU oracle, which evaluates both definitions in
fp64.  The GPU evaluates them in fp32 (its own reduction order, exp and tanh),
so its int8 codes are checked as valid roundings of the fp64 values h:

  * the scale within rel relative of max|h| / 127, and
  * every code within 0.5 + 127 * 2 * rel of h / sx, |q| <= 127,

where rel bounds the relative fp32 error of one value:
  * RMSNorm: the sum of k positive squares over 256 partials then 8 pairwise
    levels (ceil(k/256) + 8 roundings), halved by the square root, plus the
    divide, eps, root, reciprocal and the two products: (ceil(k/256) + 20) u;
  * gate: 4e-7 (a few roundings of exp / tanh and the products).
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


U = 2.0 ** -24


def _check_valid_rounding(x8, sx, h, rel):
    s_ref = np.maximum(np.abs(h).max(axis=1), 1e-9) / 127.0
    s_gpu = sx.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(s_gpu - s_ref) <= rel * s_ref), np.max(np.abs(s_gpu - s_ref) / s_ref)
    q = x8.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(q - h / s_gpu[:, None]) <= 0.5 + 127 * 2 * rel)
    assert np.all(np.abs(q) <= 127)
    return q


def _rms_rel(k):
    return ((k + 255) // 256 + 20) * U


@pytest.mark.parametrize("m,k", [(1, 1152), (4, 6912), (3, 257), (2, 1), (16, 1536), (512, 1152)])
def test_rmsnorm_quantize_valid_rounding(qmv_gpu, m, k):
    from ternary_matvec_amd import qmv
    say("rmsnorm_quantize %d x %d" % (m, k))
    x = synth.normal(91 + k, (m, k)) * 3.0
    w = synth.normal(92 + k, (k,)) * 0.3 + 1.0
    x8, sx = qmv.qmv_rmsnorm_quantize(torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV), 1e-5)
    torch.cuda.synchronize()
    _check_valid_rounding(x8, sx, oracle.rmsnorm(x, w, 1e-5), _rms_rel(k))


def test_rmsnorm_quantize_zero_row_and_eps(qmv_gpu):
    from ternary_matvec_amd import qmv
    k = 300
    tiny = synth.normal(93, (1, k)) * 1e-4
    w = np.ones(k, np.float32)
    cases = [(np.concatenate([np.zeros((1, k), np.float32), tiny]), 1e-5),
             (np.concatenate([np.zeros((1, k), np.float32), tiny]), 1e-2),
             (tiny, 0.0)]          # eps = 0 only without a zero row (0 / 0 is outside the domain)
    for x, eps in cases:
        x8, sx = qmv.qmv_rmsnorm_quantize(torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV), eps)
        torch.cuda.synchronize()
        h = oracle.rmsnorm(x, w, eps)
        q = _check_valid_rounding(x8, sx, h, _rms_rel(k))
        zero = ~np.any(x != 0, axis=1)
        assert np.all(q[zero] == 0)
        assert np.all(sx.cpu().numpy()[zero] == np.float32(np.float32(1e-9) / np.float32(127.0)))


@pytest.mark.parametrize("act", [1, 2])
@pytest.mark.parametrize("m,n", [(1, 6912), (4, 4096), (3, 1001), (512, 6912)])
def test_glu_quantize_valid_rounding(qmv_gpu, act, m, n):
    from ternary_matvec_amd import qmv
    say("glu_quantize act=%d %d x %d" % (act, m, n))
    g = synth.normal(94 + n + act, (m, n)) * 2.0
    u = synth.normal(95 + n + act, (m, n))
    g[0, :4] = [0.0, -0.0, 12.0, -12.0]
    x8, sx = qmv.qmv_glu_quantize(torch.from_numpy(g).to(DEV), torch.from_numpy(u).to(DEV), act)
    torch.cuda.synchronize()
    q = _check_valid_rounding(x8, sx, oracle.glu(g, u, act), 4e-7)
    assert np.all(q[0, :2] == 0)


def test_glu_quantize_zero_gate(qmv_gpu):
    from ternary_matvec_amd import qmv
    g = np.zeros((1, 64), np.float32)
    u = synth.normal(96, (1, 64))
    x8, sx = qmv.qmv_glu_quantize(torch.from_numpy(g).to(DEV), torch.from_numpy(u).to(DEV), 1)
    torch.cuda.synchronize()
    assert np.all(x8.cpu().numpy() == 0)
    assert sx.cpu().numpy()[0] == np.float32(np.float32(1e-9) / np.float32(127.0))
