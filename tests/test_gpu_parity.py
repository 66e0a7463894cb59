"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact for packed bytes, int8 codes, scales and int32 accumulators; fp32
outputs within 1e-6 relative of the oracle's correctly rounded value; bf16
output-layer logits within max(2e-2 |r|, gamma_K * sum|w x|) and the chosen
index equal to the oracle's unless the two logits are within that tolerance.
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


def _t(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def _x_for(seed, m, k, std=1.0):
    return synth.normal(seed, (m, k), std=std)


# --------------------------------------------------------------------------
# A1: activation quantisation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("m,k", [(1, 1), (1, 7), (2, 5), (3, 288), (130, 1152), (2, 6912), (4, 1537), (1, 70001)])
def test_quantize_act_bit_exact(qmv_gpu, m, k):
    from ternary_matvec_amd import qmv
    say("quantize_act", m, k)
    x = _x_for(1000 + k, m, k, std=2.5)
    if m > 1:
        x[1, :] = 0.0                       # zero row -> floor scale
    x[0, 0] = 127.0 if k > 1 else x[0, 0]   # keep one exact half case alive in row 0
    if k > 3:
        x[0, 1], x[0, 2], x[0, 3] = 0.5, 2.5, -2.5
    q_ref, s_ref = oracle.quantize_rows(x)
    x8, sx = qmv.qmv_quantize_act(_t(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(x8.cpu().numpy(), q_ref)


def test_quantize_act_many_bit_exact_and_equal_to_single_calls(qmv_gpu):
    from ternary_matvec_amd import qmv
    say("quantize_act_many: 4 sets of different widths in one launch")
    shapes = [(130, 1152), (26, 6912), (1, 7), (3, 1537)]
    xs = [_x_for(1500 + i, m, k, std=1.5 + i) for i, (m, k) in enumerate(shapes)]
    xs[0][5, :] = 0.0
    xd = [_t(x) for x in xs]
    outs = [(torch.full((m, k), 77, dtype=torch.int8, device=DEV), torch.zeros(m, dtype=torch.float32, device=DEV))
            for (m, k) in shapes]
    qmv.qmv_quantize_act_many([(x, o[0], o[1]) for x, o in zip(xd, outs)])
    torch.cuda.synchronize()
    for x, x_d, (x8, sx) in zip(xs, xd, outs):
        q_ref, s_ref = oracle.quantize_rows(x)
        np.testing.assert_array_equal(x8.cpu().numpy(), q_ref)
        np.testing.assert_array_equal(sx.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
        x8s, sxs = qmv.qmv_quantize_act(x_d)
        torch.cuda.synchronize()
        assert torch.equal(x8s, x8) and torch.equal(sxs.view(torch.int32), sx.view(torch.int32))


def test_quantize_act_unaligned_rows(qmv_gpu):
    from ternary_matvec_amd import qmv
    say("quantize_act unaligned")
    x = _x_for(77, 5, 33)
    big = torch.zeros(5 * 33 + 1, dtype=torch.float32, device=DEV)
    big[1:] = _t(x).reshape(-1)
    xin = big[1:].view(5, 33)                      # 4-byte aligned, not 16-byte aligned
    x8 = torch.empty(5 * 33 + 3, dtype=torch.int8, device=DEV)[3:].view(5, 33)
    sx = torch.empty(5, dtype=torch.float32, device=DEV)
    qmv.qmv_quantize_act(xin, x8=x8, sx=sx)
    q_ref, s_ref = oracle.quantize_rows(x)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(x8.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(sx.cpu().numpy(), s_ref)


# --------------------------------------------------------------------------
# A10: packing
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(1, 1), (3, 7), (9, 23), (64, 81), (300, 1152), (17, 6912), (65, 160)])
def test_pack_ternary_bit_exact(qmv_gpu, n, k):
    from ternary_matvec_amd import qmv
    say("pack_ternary", n, k)
    t = synth.trits(2000 + k, (n, k))
    ref, bad = oracle.pack_trit5(t)
    bad_dev = torch.full((1,), 77, dtype=torch.int32, device=DEV)
    w = qmv.qmv_pack_ternary(_t(t), 0.0173, bad_count=bad_dev)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w.packed.cpu().numpy(), ref)
    assert w.scale.item() == np.float32(0.0173)
    assert bad_dev.item() == bad == 0
    assert w.n == n and w.k == k and w.wtype == qmv.QMV_W_TERNARY5


def test_pack_ternary_counts_bad_trits(qmv_gpu):
    from ternary_matvec_amd import qmv
    say("pack_ternary bad trits")
    t = synth.trits(31, (40, 50))
    t[3, 4], t[17, 0], t[39, 49] = 2, -5, 100
    ref, bad = oracle.pack_trit5(t)
    bad_dev = torch.zeros(1, dtype=torch.int32, device=DEV)
    w = qmv.qmv_pack_ternary(_t(t), 1.0, bad_count=bad_dev)
    torch.cuda.synchronize()
    assert bad == 3 and bad_dev.item() == 3
    np.testing.assert_array_equal(w.packed.cpu().numpy(), ref)


@pytest.mark.parametrize("n,k", [(768, 288), (5, 17), (1, 1), (33, 100)])
def test_pack_int8_bit_exact(qmv_gpu, n, k):
    from ternary_matvec_amd import qmv
    say("pack_int8", n, k)
    w = synth.normal(3000 + k, (n, k), std=0.02)
    q_ref, s_ref = oracle.quantize_tensor(w)
    ref = oracle.layout_int8(q_ref)
    pw = qmv.qmv_pack_int8(_t(w))
    torch.cuda.synchronize()
    assert pw.scale.cpu().numpy().view(np.uint32)[0] == np.float32(s_ref).view(np.uint32)
    np.testing.assert_array_equal(pw.packed.cpu().numpy().view(np.int8), ref)


# --------------------------------------------------------------------------
# A2-A7: GEMV
# --------------------------------------------------------------------------

def _check_y(y, acc_ref, sx, sw):
    y_ref = oracle.dequant(acc_ref, sx, sw)
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    tol = 1e-6 * np.abs(y_ref.astype(np.float64))
    assert np.all(err <= tol), float((err - tol).max())
    assert np.all(y[acc_ref == 0] == 0.0)


# (n, k, m): ragged rows and columns, every lanes-per-row split of the
# streaming kernel (row chunks 1..32, 33..64, 65+; odd chunk counts leave
# lanes with one chunk less), and the workgroup kernel for m > 2.
GEMV_CASES = [(1, 1, 1), (5, 7, 1), (64, 80, 1), (65, 81, 2), (3, 400, 1), (200, 1152, 1), (130, 1152, 3),
              (1152, 6912, 1), (77, 6912, 2), (100, 2800, 1), (50, 5000, 2), (33, 4096, 1), (100, 1000, 16),
              (64, 5, 4), (257, 333, 8), (70, 1600, 5), (17, 6912, 4)]


@pytest.mark.parametrize("dot_only", [False, True], ids=["mfma", "dot"])
@pytest.mark.parametrize("n,k,m", GEMV_CASES)
def test_gemv_ternary_parity(qmv_gpu, n, k, m, dot_only):
    from ternary_matvec_amd import qmv
    say("gemv ternary", n, k, m, "dot only" if dot_only else "matrix cores")
    t = synth.trits(4000 + n + k, (n, k))
    x = _x_for(5000 + k + m, m, k)
    q, sx = oracle.quantize_rows(x)
    sw = synth.ternary_scale(6000 + n)
    acc_ref = oracle.matmul_int(q, t)
    w = qmv.qmv_pack_ternary(_t(t), sw)
    acc = torch.full((m, n), -7, dtype=torch.int32, device=DEV)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    p = qmv.Problem(w, _t(q), _t(sx), y=y, acc=acc)
    qmv.gemv_plan([p], dot_only=dot_only).launch()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    _check_y(p.y.cpu().numpy(), acc_ref, sx, np.float32(sw))


@pytest.mark.parametrize("n,k,m", [(768, 288, 1), (33, 17, 3), (64, 4096, 2), (5, 1, 16), (40, 1040, 1), (9, 700, 2)])
def test_gemv_int8_parity(qmv_gpu, n, k, m):
    from ternary_matvec_amd import qmv
    say("gemv int8", n, k, m)
    wf = synth.normal(7000 + k, (n, k), std=0.02)
    q_w, s_w = oracle.quantize_tensor(wf)
    x = _x_for(7100 + k, m, k)
    q, sx = oracle.quantize_rows(x)
    acc_ref = oracle.matmul_int(q, q_w)
    pw = qmv.qmv_pack_int8(_t(wf))
    acc = torch.zeros((m, n), dtype=torch.int32, device=DEV)
    p = qmv.Problem(pw, _t(q), _t(sx), acc=acc)
    qmv.qmv_gemv([p])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    _check_y(p.y.cpu().numpy(), acc_ref, sx, s_w)


def test_gemv_grouped_mixed_equals_single(qmv_gpu):
    """One grouped launch over ternary and int8 problems of mixed shapes and
    token counts gives the same bits as one launch per problem."""
    from ternary_matvec_amd import qmv
    say("gemv grouped mixed")
    specs = [(1, 1024, 1152, 1), (1, 256, 1152, 2), (2, 100, 288, 1), (1, 1152, 6912, 1), (2, 64, 80, 3),
             (1, 6912, 1152, 1), (1, 7, 9, 16)]
    probs, refs = [], []
    for i, (wt, n, k, m) in enumerate(specs):
        x = _x_for(8000 + i, m, k)
        q, sx = oracle.quantize_rows(x)
        if wt == 1:
            t = synth.trits(8100 + i, (n, k))
            w = qmv.qmv_pack_ternary(_t(t), 0.02 + i * 1e-3)
            refs.append(oracle.matmul_int(q, t))
        else:
            wf = synth.normal(8200 + i, (n, k), std=0.05)
            w = qmv.qmv_pack_int8(_t(wf))
            refs.append(oracle.matmul_int(q, oracle.quantize_tensor(wf)[0]))
        probs.append(qmv.Problem(w, _t(q), _t(sx), acc=torch.zeros((m, n), dtype=torch.int32, device=DEV)))
    plan = qmv.gemv_plan(probs)
    plan.launch()
    torch.cuda.synchronize()
    grouped = [(p.acc.cpu().numpy().copy(), p.y.cpu().numpy().copy()) for p in probs]
    for p, ref, (acc_g, y_g) in zip(probs, refs, grouped):
        np.testing.assert_array_equal(acc_g, ref)
        p.acc.zero_()
        p.y.zero_()
        qmv.qmv_gemv([p])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(p.acc.cpu().numpy(), acc_g)
        np.testing.assert_array_equal(p.y.cpu().numpy(), y_g)
    # a second launch of the plan (its table uploaded once) gives the same bits
    for p in probs:
        p.y.zero_()
    plan.launch()
    torch.cuda.synchronize()
    for p, (_, y_g) in zip(probs, grouped):
        np.testing.assert_array_equal(p.y.cpu().numpy(), y_g)


def test_plan_launch_in_a_graph_and_one_shot_refused_under_capture(qmv_gpu):
    """A plan's launch (kernels only) captured in a HIP graph and replayed,
    with eager work between the replays, gives the eager result every time;
    the one-shot qmv_gemv refuses a capturing stream (its upload would keep a
    pointer to released host memory) and enqueues nothing."""
    from ternary_matvec_amd import qmv
    say("plan launch in a graph")
    specs = [(1024, 1152, 1), (256, 1152, 1), (1152, 6912, 1), (6912, 1152, 1)]
    probs, refs = [], []
    for i, (n, k, m) in enumerate(specs):
        t = synth.trits(8300 + i, (n, k))
        q, sx = oracle.quantize_rows(_x_for(8400 + i, m, k))
        w = qmv.qmv_pack_ternary(_t(t), 0.02)
        refs.append(oracle.matmul_int(q, t))
        probs.append(qmv.Problem(w, _t(q), _t(sx), acc=torch.zeros((m, n), dtype=torch.int32, device=DEV)))
    plan = qmv.gemv_plan(probs)
    plan.launch()
    torch.cuda.synchronize()
    eager = [p.y.clone() for p in probs]
    for p, ref in zip(probs, refs):
        np.testing.assert_array_equal(p.acc.cpu().numpy(), ref)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    refused = None
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            plan.launch(cap)
            try:
                qmv.qmv_gemv(probs, stream=cap)
            except qmv.QmvError as e:
                refused = e.status
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    assert refused == qmv.QMV_EUNSUPPORTED
    for _ in range(3):
        for p in probs:
            p.y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for p, e in zip(probs, eager):
            assert torch.equal(p.y, e)
        plan.launch()                      # eager work between the replays
        torch.cuda.synchronize()


# Zero-group skipping (QMV_PLAN_GEMV_SKIP_ZERO): activations with 80% of their
# groups of 4 columns zero, all zero, or dense; one and two tokens (a unit is
# skipped only when it is zero for both); row lengths that give every
# lanes-per-row split (the skip must hold for all chunks of a step).  Exact:
# acc equals the oracle's and y equals the dense plan's bit for bit.
SKIP_CASES = [(200, 1152, 1), (1152, 6912, 1), (77, 6912, 2), (100, 2800, 1), (5, 7, 1), (64, 80, 2),
              (300, 1536, 2), (33, 4096, 1)]


@pytest.mark.parametrize("density", ["sparse", "zero", "dense", "mixed"])
@pytest.mark.parametrize("n,k,m", SKIP_CASES)
def test_gemv_skip_zero_parity(qmv_gpu, n, k, m, density):
    from ternary_matvec_amd import qmv
    say("gemv skip zero", n, k, m, density)
    t = synth.trits(15000 + n + k, (n, k))
    x = _x_for(15001 + k + m, m, k)
    if density == "sparse":
        x[synth.zero_groups(15002 + k, x.shape)] = 0.0
    elif density == "zero":
        x[:] = 0.0
    elif density == "mixed":          # token 0 sparse, token 1 (if any) dense
        x[0][synth.zero_groups(15003 + k, (k,))] = 0.0
    q, sx = oracle.quantize_rows(x)
    sw = synth.ternary_scale(15004 + n)
    acc_ref = oracle.matmul_int(q, t)
    w = qmv.qmv_pack_ternary(_t(t), sw)
    acc = torch.full((m, n), -7, dtype=torch.int32, device=DEV)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    p = qmv.Problem(w, _t(q), _t(sx), y=y, acc=acc)
    qmv.gemv_plan([p], skip_zero=True).launch()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    _check_y(y.cpu().numpy(), acc_ref, sx, np.float32(sw))
    y_skip = y.clone()
    y.fill_(float("nan"))
    qmv.gemv_plan([p]).launch()
    torch.cuda.synchronize()
    assert torch.equal(y, y_skip)


def test_gemv_skip_zero_grouped_launch(qmv_gpu):
    """One skip-plan launch over mixed shapes (every lanes-per-row split in one
    table), launched twice, equals the oracle exactly."""
    from ternary_matvec_amd import qmv
    say("gemv skip zero grouped")
    specs = [(1024, 1152, 1), (256, 1152, 1), (6912, 1152, 1), (1152, 6912, 1), (100, 333, 1)]
    probs, refs = [], []
    for i, (n, k, m) in enumerate(specs):
        t = synth.trits(15100 + i, (n, k))
        x = _x_for(15200 + i, m, k)
        x[synth.zero_groups(15300 + i, x.shape)] = 0.0
        q, sx = oracle.quantize_rows(x)
        refs.append(oracle.matmul_int(q, t))
        probs.append(qmv.Problem(qmv.qmv_pack_ternary(_t(t), 0.02), _t(q), _t(sx),
                                 acc=torch.zeros((m, n), dtype=torch.int32, device=DEV)))
    plan = qmv.gemv_plan(probs, skip_zero=True)
    for _ in range(2):
        for p in probs:
            p.acc.fill_(-7)
        plan.launch()
        torch.cuda.synchronize()
        for p, ref in zip(probs, refs):
            np.testing.assert_array_equal(p.acc.cpu().numpy(), ref)


def test_gemv_batch_columns_equal_single_token(qmv_gpu):
    """Exact integers: token j of a 16-token problem equals the 1-token result."""
    from ternary_matvec_amd import qmv
    say("gemv batch invariance")
    n, k, m = 300, 1536, 16
    t = synth.trits(9000, (n, k))
    q, sx = oracle.quantize_rows(_x_for(9001, m, k))
    w = qmv.qmv_pack_ternary(_t(t), 0.02)
    acc16 = torch.zeros((m, n), dtype=torch.int32, device=DEV)
    qmv.qmv_gemv([qmv.Problem(w, _t(q), _t(sx), acc=acc16)])
    for j in (0, 5, 15):
        acc1 = torch.zeros((1, n), dtype=torch.int32, device=DEV)
        qmv.qmv_gemv([qmv.Problem(w, _t(q[j:j + 1]), _t(sx[j:j + 1]), acc=acc1)])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc1.cpu().numpy()[0], acc16.cpu().numpy()[j])


def test_gemv_extreme_values(qmv_gpu):
    """All +1 / all -1 / one-hot rows against activations at the int8 extremes."""
    from ternary_matvec_amd import qmv
    say("gemv extremes")
    k = 6912
    t = np.zeros((64 + 3, k), np.int8)
    t[0] = 1
    t[1] = -1
    for r in range(2, 67):
        t[r, (r * 101) % k] = 1 if r % 2 else -1
    q = np.full((2, k), -128, np.int8)
    q[1] = 127
    sx = np.array([0.5, 0.25], np.float32)
    acc_ref = oracle.matmul_int(q, t)
    w = qmv.qmv_pack_ternary(_t(t), 1.0)
    acc = torch.zeros((2, t.shape[0]), dtype=torch.int32, device=DEV)
    qmv.qmv_gemv([qmv.Problem(w, _t(q), _t(sx), acc=acc)])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    assert acc_ref[0, 0] == -128 * k and acc_ref[1, 1] == -127 * k


# --------------------------------------------------------------------------
# A9: output layer + greedy choice
# --------------------------------------------------------------------------

def _check_head(w_bits, x, idx, logits):
    ref, ref_idx = oracle.lmhead(w_bits, x)
    wf = synth.bf16_bits_to_f32(w_bits).astype(np.float64)
    k = x.size
    gamma = k * 2.0 ** -24 / (1 - k * 2.0 ** -24)
    absdot = np.abs(wf) @ np.abs(x.astype(np.float64))
    tol = np.maximum(2e-2 * np.abs(ref), gamma * absdot)
    if logits is not None:
        err = np.abs(logits.astype(np.float64) - ref)
        assert np.all(err <= tol), float((err - tol).max())
    if idx != ref_idx:
        assert abs(ref[idx] - ref[ref_idx]) <= max(tol[idx], tol[ref_idx]), (idx, ref_idx)
    return ref_idx


@pytest.mark.parametrize("v,k", [(1, 8), (100, 64), (1000, 1152), (5000, 1000), (333, 2050), (64, 9)])
def test_lmhead_parity(qmv_gpu, v, k):
    from ternary_matvec_amd import qmv
    say("lmhead", v, k)
    w_bits = synth.to_bf16_bits(synth.normal(10000 + v, (v, k), std=0.02))
    x = synth.normal(10001 + k, (k,))
    idx, mx, logits = qmv.qmv_lmhead_argmax(_t(w_bits.view(np.int16)), _t(x), want_logits=True)
    torch.cuda.synchronize()
    _check_head(w_bits, x, int(idx.item()), logits.cpu().numpy())
    assert mx.item() == logits.cpu().numpy()[int(idx.item())]


def test_lmhead_planted_winner_and_tie(qmv_gpu):
    from ternary_matvec_amd import qmv
    say("lmhead planted")
    v, k = 20000, 1152
    w_bits = synth.to_bf16_bits(synth.normal(11000, (v, k), std=0.02))
    x = synth.normal(11001, (k,))
    w_bits[12345] = synth.to_bf16_bits(np.sign(x) * 0.5)
    idx, _, _ = qmv.qmv_lmhead_argmax(_t(w_bits.view(np.int16)), _t(x))
    torch.cuda.synchronize()
    assert idx.item() == 12345
    w_bits[777] = w_bits[12345]                       # an exact tie: the first index wins
    w_bits[19999] = w_bits[12345]
    idx, _, _ = qmv.qmv_lmhead_argmax(_t(w_bits.view(np.int16)), _t(x))
    torch.cuda.synchronize()
    assert idx.item() == 777


# --------------------------------------------------------------------------
# A8: prefill GEMM on int8 matrix cores
# --------------------------------------------------------------------------

# (n, k, m): ragged tokens and rows around the 128-token x 256-row tile, odd
# chunk counts (the last K step is half empty), K not a multiple of 4 or 16
# (activation rows staged byte-wise), a single K step.
PREFILL_CASES = [(1, 1, 1), (5, 7, 3), (64, 80, 32), (300, 1152, 256), (257, 1152, 300), (33, 6912, 512),
                 (1024, 1152, 512), (100, 1600, 17), (513, 161, 257), (40, 1537, 5), (256, 1152, 128),
                 (255, 1152, 129), (260, 1160, 127), (768, 2304, 384)]


@pytest.mark.parametrize("n,k,m", PREFILL_CASES)
def test_prefill_parity(qmv_gpu, n, k, m):
    from ternary_matvec_amd import qmv
    say("prefill", n, k, m)
    t = synth.trits(12000 + n + k, (n, k))
    x = _x_for(12001 + k + m, m, k)
    q, sx = oracle.quantize_rows(x)
    sw = synth.ternary_scale(12002 + n)
    acc_ref = oracle.matmul_int(q, t)
    w = qmv.qmv_pack_ternary(_t(t), sw)
    acc = torch.full((m, n), -7, dtype=torch.int32, device=DEV)
    p = qmv.Problem(w, _t(q), _t(sx), acc=acc)
    qmv.qmv_gemm_prefill([p])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
    _check_y(p.y.cpu().numpy(), acc_ref, sx, np.float32(sw))


# acc = NULL: the epilogue that stores y alone (buffer stores for whole tiles),
# the path the benchmark's prefill takes.  Full 128-token x 256-row tiles,
# ragged edges in tokens and rows, a single K step, every element checked
# (y starts as NaN, so an element never written fails).
PREFILL_NOACC_CASES = [(512, 1152, 256), (1000, 1152, 300), (256, 6912, 128), (300, 161, 129), (1, 1, 1),
                       (6912, 1152, 512), (257, 80, 5)]


@pytest.mark.parametrize("n,k,m", PREFILL_NOACC_CASES)
def test_prefill_parity_y_only(qmv_gpu, n, k, m):
    from ternary_matvec_amd import qmv
    say("prefill y only", n, k, m)
    t = synth.trits(12500 + n + k, (n, k))
    x = _x_for(12501 + k + m, m, k)
    q, sx = oracle.quantize_rows(x)
    sw = synth.ternary_scale(12502 + n)
    acc_ref = oracle.matmul_int(q, t)
    w = qmv.qmv_pack_ternary(_t(t), sw)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
    p = qmv.Problem(w, _t(q), _t(sx), y=y)
    qmv.qmv_gemm_prefill([p])
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert not np.isnan(got).any()
    _check_y(got, acc_ref, sx, np.float32(sw))


def test_prefill_grouped_equals_gemv(qmv_gpu):
    """Grouped prefill over mixed shapes equals single launches, and each
    token row equals the decode GEMV of that token (exact integers)."""
    from ternary_matvec_amd import qmv
    say("prefill grouped vs gemv")
    specs = [(1024, 1152, 40), (256, 1152, 7), (1152, 6912, 3), (6912, 1152, 2)]
    probs, refs, ins = [], [], []
    for i, (n, k, m) in enumerate(specs):
        t = synth.trits(13000 + i, (n, k))
        q, sx = oracle.quantize_rows(_x_for(13100 + i, m, k))
        w = qmv.qmv_pack_ternary(_t(t), 0.02)
        refs.append(oracle.matmul_int(q, t))
        ins.append((w, q, sx))
        probs.append(qmv.Problem(w, _t(q), _t(sx), acc=torch.zeros((m, n), dtype=torch.int32, device=DEV)))
    qmv.qmv_gemm_prefill(probs)
    torch.cuda.synchronize()
    for p, ref, (w, q, sx) in zip(probs, refs, ins):
        got = p.acc.cpu().numpy()
        np.testing.assert_array_equal(got, ref)
        y_grouped = p.y.cpu().numpy().copy()
        single = qmv.Problem(w, _t(q), _t(sx), acc=torch.zeros_like(p.acc))
        qmv.qmv_gemm_prefill([single])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(single.y.cpu().numpy(), y_grouped)
        for j in (0, q.shape[0] - 1):
            one = qmv.Problem(w, _t(q[j:j + 1]), _t(sx[j:j + 1]), acc=torch.zeros((1, w.n), dtype=torch.int32, device=DEV))
            qmv.qmv_gemv([one])
            torch.cuda.synchronize()
            np.testing.assert_array_equal(one.acc.cpu().numpy()[0], got[j])
