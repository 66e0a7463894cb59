"""GPU parity of the sketch head (qmv_sketch_build + qmv_lmhead_sketch_argmax)
against the CPU oracle.

  * the built tables: every sign word, every element of the dimension-major
    copy and the table scale c, bit-exact;
  * the approximate scores of steps 1 and 2, bit-exact (both sides use the
    same fp32 operation order, so the candidate set is the same);
  * the candidate count, exactly;
  * the pick: the oracle's pick, or a candidate whose exact logit is within
    the fp32 summation bound of it (the GPU sums logits in fp32, the oracle
    in fp64), and max_logit within that bound of the oracle's logit.
Shapes: small and ragged cases, fewer words than 1024, k <= 32 (all exact),
ties, and the output layer's full 262144 x 1152.
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


def _round(n, a):
    return (n + a - 1) // a * a


def _tables(sketch, v, k):
    raw = sketch.cpu().numpy()
    kw = (k + 31) // 32
    c = raw[16:20].view(np.float32)[0]
    signs = raw[256:256 + 4 * kw * v].view(np.uint32).reshape(kw, v)
    off = 256 + _round(4 * kw * v, 256)
    wt = raw[off:off + 2 * k * v].view(np.uint16).reshape(k, v)
    return c, signs, wt


def _tol(w_bits, x, rows):
    k = x.size
    wf = synth.bf16_bits_to_f32(w_bits[rows]).astype(np.float64)
    gamma = k * 2.0 ** -24 / (1 - k * 2.0 ** -24)
    return gamma * (np.abs(wf) @ np.abs(x.astype(np.float64)))


def _run(w_bits, x, build_check=True, calls=1):
    from ternary_matvec_amd import qmv
    v, k = w_bits.shape
    w = torch.from_numpy(w_bits.view(np.int16)).to(DEV)
    sketch = qmv.qmv_sketch_build(w)
    torch.cuda.synchronize()
    c_ref = oracle.sketch_scale(w_bits)
    c, signs, wt = _tables(sketch, v, k)
    assert c == c_ref, (c, c_ref)
    if build_check:
        np.testing.assert_array_equal(signs, oracle.sketch_signs(w_bits))
        np.testing.assert_array_equal(wt, w_bits.T)
    xd = torch.from_numpy(x).to(DEV)
    ws = qmv._alloc_aligned(qmv.qmv_sketch_workspace_bytes(v, k), xd.device)
    for _ in range(calls):
        idx, mx, ncand, scores = qmv.qmv_lmhead_sketch_argmax(w, sketch, xd, workspace=ws, want_scores=True)
    torch.cuda.synchronize()
    s_ref = oracle.sketch_scores(w_bits, x, c_ref)
    np.testing.assert_array_equal(scores.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    cand, logits, idx_ref = oracle.sketch_pick(w_bits, x, s_ref)
    assert int(ncand.item()) == int(cand.sum())
    i = int(idx.item())
    assert cand[i]
    tol = _tol(w_bits, x, np.array([i, idx_ref]))
    if i != idx_ref:
        assert abs(logits[i] - logits[idx_ref]) <= max(tol), (i, idx_ref, logits[i], logits[idx_ref])
    assert abs(float(mx.item()) - logits[i]) <= tol[0] + 1e-30
    return i, idx_ref, cand


@pytest.mark.parametrize("v,k", [(3000, 96), (2500, 40), (4099, 1152), (1500, 8), (1100, 264)])
def test_sketch_small_shapes(qmv_gpu, v, k):
    say("sketch %d x %d" % (v, k))
    w = synth.to_bf16_bits(synth.normal(1000 + k, (v, k), std=0.02))
    x = synth.normal(2000 + k, (k,))
    _run(w, x)


def test_sketch_fewer_words_than_candidates(qmv_gpu):
    say("sketch 700 x 128: every word a candidate")
    w = synth.to_bf16_bits(synth.normal(71, (700, 128), std=0.02))
    x = synth.normal(72, (128,))
    i, ref, cand = _run(w, x)
    assert cand.all()
    w1 = w[:1].copy()
    i1, _, _ = _run(w1, x)
    assert i1 == 0


def test_sketch_all_dimensions_exact(qmv_gpu):
    say("sketch 5000 x 32: k <= 32 scores everything exactly")
    w = synth.to_bf16_bits(synth.normal(73, (5000, 32), std=0.02))
    x = synth.normal(74, (32,))
    i, ref, _ = _run(w, x)
    full, fidx = oracle.lmhead(w, x)
    assert ref == fidx


def test_sketch_ties_planted_winner_and_repeat_calls(qmv_gpu):
    say("sketch 20000 x 1152: planted winner, duplicate rows, equal |x|, two calls")
    v, k = 20000, 1152
    w = synth.to_bf16_bits(synth.normal(75, (v, k), std=0.02))
    wf = synth.bf16_bits_to_f32(w)
    x = (40.0 * wf[12345] + synth.normal(76, (k,)) * 0.2).astype(np.float32)
    w[777] = w[12345]                                   # tie: the lower index wins
    i, ref, cand = _run(w, x, calls=2)
    assert i == ref == 777
    xe = np.where(synth.raw(77, k) % 2 == 0, 1.0, -1.0).astype(np.float32)   # all |x| equal
    _run(w, xe, build_check=False)


def test_sketch_fullsize_output_layer(qmv_gpu):
    say("sketch 262144 x 1152 (the output layer), 3 tokens")
    v, k = synth.HEAD_V, synth.HEAD_K
    w0 = synth.normal_torch(synth.stream_seed(synth.CONFIG_HEAD, 0, 0, synth.TAG_HEAD), (v, k), std=0.02, device=DEV)
    w_bits = w0.to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    del w0
    torch.cuda.empty_cache()
    for t in range(3):
        x = synth.normal(synth.stream_seed(synth.CONFIG_HEAD, 1, t, synth.TAG_ACT), (k,))
        _run(w_bits, x, build_check=(t == 0))
