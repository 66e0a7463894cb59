"""GPU parity of the sketch head (qmv_sketch_build + qmv_lmhead_sketch_argmax)
against the CPU oracle, which evaluates the page's definition in fp64 and takes
the plain N = min(1024, v) best approximate scores as its candidates.

  * the built tables: every sign word and every element of the
    dimension-major copy bit-exact; c within the fp32 bound of its
    summation (all terms positive: (k + 1) roundings relative);
  * the approximate scores within the bound of their fp32 evaluation:
    (T + 4) roundings of the fused multiply-add chain plus the relative error
    of the group weights ((k + n_g + 2) roundings), times the sum of the
    magnitudes of the score's terms;
  * the GPU's candidates, rebuilt from its own scores by its documented rule
    (the top bins of 13-bit order keys that hold at least N words, among the
    256 bins below the highest non-empty one, else every word), number
    what the kernel reports, and contain every word whose oracle score clears
    the N-th best upper bound by more than its own error bound
    (containment: such a word is in the GPU's top N whatever the rounding);
  * the pick: a GPU candidate whose exact logit (fp64) is within the fp32
    summation bound of the best exact logit among the GPU's candidates, and
    of the oracle's pick whenever that word is surely a GPU candidate;
    max_logit within that bound of the pick's exact logit.
Shapes: small and ragged cases, fewer words than 1024, k <= 32 (all exact),
ties, the output layer's full 262144 x 1152, and 300000 rows (more workgroups
than compute units).  The workspace carries state
from call to call: one workspace is also reused over several shapes in a row.
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


BIN_BITS = 13      # the candidate rule's bins: top 13 bits of the score's order key
WINDOW = 256       # bins searched below the highest non-empty one


def _tables(sketch, v, k):
    """The header's c, the sign words [kw][vp] and the copy [k][vp], vp = v rounded up to 1024."""
    raw = sketch.cpu().numpy()
    kw = (k + 31) // 32
    vp = _round(v, 1024)
    c = raw[16:20].view(np.float32)[0]
    signs = raw[256:256 + 4 * kw * vp].view(np.uint32).reshape(kw, vp)
    off = 256 + _round(4 * kw * vp, 256)
    wt = raw[off:off + 2 * k * vp].view(np.uint16).reshape(k, vp)
    return c, signs, wt


U = 2.0 ** -24


def _tol(w_bits, x, rows):
    k = x.size
    wf = synth.bf16_bits_to_f32(w_bits[rows]).astype(np.float64)
    gamma = k * U / (1 - k * U)
    return gamma * (np.abs(wf) @ np.abs(x.astype(np.float64)))


def _score_bound(k, group_n, mag):
    t = min(32, k)
    rel = ((t + 4) + (k + int(max(group_n)) + 2)) * U * 1.01
    return rel * mag + 1e-30


def _bins(scores32):
    u = scores32.view(np.uint32).astype(np.uint64)
    return (np.where(u & 0x80000000, ~u & 0xFFFFFFFF, u | 0x80000000) >> (32 - BIN_BITS)).astype(np.int64)


def _gpu_candidates(scores32, n_need):
    """The documented rule: the top bins (13-bit order keys) holding at least n_need words,
    searched over the WINDOW bins below the highest non-empty one; every word if those hold fewer."""
    nb = 1 << BIN_BITS
    b = _bins(scores32)
    in_window = b >= b.max() - (WINDOW - 1)
    hist = np.bincount(b[in_window], minlength=nb)
    above = np.cumsum(hist[::-1])
    if above[-1] < n_need:
        return np.ones(b.shape, dtype=bool)
    bstar = nb - 1 - int(np.argmax(above >= n_need))
    return b >= bstar


def _run(w_bits, x, build_check=True, calls=1, ws=None):
    from ternary_matvec_amd import qmv
    v, k = w_bits.shape
    w = torch.from_numpy(w_bits.view(np.int16)).to(DEV)
    sketch = qmv.qmv_sketch_build(w)
    torch.cuda.synchronize()
    c_ref = oracle.sketch_scale(w_bits)
    c, signs, wt = _tables(sketch, v, k)
    assert abs(float(c) - c_ref) <= (k + 1) * U * 1.01 * c_ref, (c, c_ref)
    if build_check:
        np.testing.assert_array_equal(signs[:, :v], oracle.sketch_signs(w_bits))
        np.testing.assert_array_equal(wt[:, :v], w_bits.T)
        assert not signs[:, v:].any() and not wt[:, v:].any()
    xd = torch.from_numpy(x).to(DEV)
    if ws is None:
        ws = qmv.sketch_workspace(v, k, xd.device)
    for _ in range(calls):
        idx, mx, ncand, scores = qmv.qmv_lmhead_sketch_argmax(w, sketch, xd, workspace=ws, want_scores=True)
    torch.cuda.synchronize()
    s_ref, mag = oracle.sketch_scores(w_bits, x, c_ref)
    _, _, group_n, _ = oracle.sketch_plan(x, c_ref)
    err = _score_bound(k, group_n, mag)
    s_gpu = scores.cpu().numpy()
    bad = np.flatnonzero(np.abs(s_gpu.astype(np.float64) - s_ref) > err)
    assert bad.size == 0, (bad[:5], s_gpu[bad[:5]], s_ref[bad[:5]], err[bad[:5]])
    n_need = min(1024, v)
    cand = _gpu_candidates(s_gpu, n_need)
    assert int(ncand.item()) == int(cand.sum()) >= n_need
    upper = np.sort(s_ref + err)[::-1][n_need - 1]
    sure = (s_ref - err) > upper
    missing = np.flatnonzero(sure & ~cand)
    assert missing.size == 0, missing[:5]
    ref_cand, ref_logits, idx_ref = oracle.sketch_pick(w_bits, x, s_ref)
    assert int(ref_cand.sum()) == n_need
    i = int(idx.item())
    assert cand[i], i
    rows = np.flatnonzero(cand)
    logits, _ = oracle.lmhead(w_bits[rows], x)
    tol_all = _tol(w_bits, x, rows)
    j = int(np.argmax(logits))
    li = float(logits[np.searchsorted(rows, i)])
    tol_i = float(tol_all[np.searchsorted(rows, i)])
    assert li >= logits[j] - tol_i - tol_all[j], (i, rows[j], li, logits[j])
    if sure[idx_ref]:
        tol = _tol(w_bits, x, np.array([i, idx_ref]))
        assert li >= ref_logits[idx_ref] - tol.sum(), (i, idx_ref, li, ref_logits[idx_ref])
    assert abs(float(mx.item()) - li) <= tol_i + 1e-30
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
    tol = _tol(w, x, np.array([i, fidx]))
    assert full[i] >= full[fidx] - tol.sum()


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


def test_sketch_workspace_reused_over_shapes(qmv_gpu):
    """One zero-filled workspace, sized for the largest shape, through tokens of
    different shapes in a row (the state each call leaves must suit any next one)."""
    from ternary_matvec_amd import qmv
    shapes = [(5000, 256), (1500, 64), (20000, 1152), (900, 96), (5000, 256)]
    ws = qmv.sketch_workspace(max(v for v, _ in shapes), max(k for _, k in shapes), DEV)
    for i, (v, k) in enumerate(shapes):
        say("sketch %d x %d on a shared workspace (call %d)" % (v, k, i))
        w = synth.to_bf16_bits(synth.normal(3000 + i, (v, k), std=0.02))
        x = synth.normal(4000 + i, (k,))
        _run(w, x, build_check=False, calls=2, ws=ws)


def test_sketch_more_workgroups_than_compute_units(qmv_gpu):
    """300000 rows = 293 workgroups of 1024 rows, more than the 256 compute units
    (several workgroups per histogram copy and exit set beyond one round); twice, so
    the state the first call leaves is used again."""
    say("sketch 300000 x 64, two calls")
    w = synth.to_bf16_bits(synth.normal(91, (300000, 64), std=0.02))
    x = synth.normal(92, (64,))
    _run(w, x, calls=2)


def test_sketch_widest_rows(qmv_gpu):
    """k = 8192, the largest supported: the bins of the top 11 bits of |x| hold more than
    64 dimensions, so the further 10-bit digits are taken, and the sign words run past
    the ones loaded before the plan."""
    say("sketch 3000 x 8192")
    w = synth.to_bf16_bits(synth.normal(95, (3000, 8192), std=0.02))
    x = synth.normal(96, (8192,))
    _run(w, x)


def test_sketch_zero_heavy_hidden_state(qmv_gpu):
    """60% of x exactly zero (some of them -0.0): the group boundaries fall among equal |x|,
    which are ranked by index."""
    say("sketch 20000 x 1152, 60% zero x")
    w = synth.to_bf16_bits(synth.normal(97, (20000, 1152), std=0.02))
    x = synth.normal(98, (1152,))
    r = synth.raw(99, 1152) % 10
    x[r < 6] = 0.0
    x[r == 0] = -0.0
    _run(w, x.astype(np.float32))
