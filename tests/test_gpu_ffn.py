"""GPU parity of qmv_ffn_decode, the feed-forward half of a layer stack for one
token in one persistent launch (llama2.c tour, "forward": Step 5 and the
residual connection; gemma.cpp tour, "The Forward Pass, Layer by Layer").

  * Bit for bit against the chain of existing entry points that defines it:
    qmv_rmsnorm_quantize -> qmv_gemv (gate, up) -> qmv_glu_quantize ->
    qmv_gemv (down) -> fp32 add, layer after layer (ragged shapes, both gates,
    more layers than one launch holds, the largest hidden and inter sizes, the
    full 26-layer Gemma-3-1B stack).
  * That chain, layer by layer, against the oracle: the int8 codes are valid
    roundings of the fp64 RMSNorm / GLU values, the int32 dots are exact, the
    dequantised outputs are within three fp32 roundings of their fp64 values,
    and h moves by exactly one fp32 add.
  * The launch's waits: a preset cancel word (device or pinned host memory)
    stops it with QMV_FFN_CANCELLED and h unchanged; a one-poll spin limit ends
    in QMV_FFN_OK or QMV_FFN_TIMEOUT; either way the workspace is left clean and
    the next call is exact.  Graph replays equal the eager call.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from ternary_matvec_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U = 2.0 ** -24


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


class Stack:
    """nlayers feed-forward layers of random ternary weights (and their trits)."""

    def __init__(self, qmv, hidden, inter, nlayers, seed, keep_trits=False):
        self.hidden, self.inter, self.nlayers = hidden, inter, nlayers
        self.layers = []
        self.trits = []
        for l in range(nlayers):
            ws = []
            tl = []
            for mi, (n, k) in enumerate(((inter, hidden), (inter, hidden), (hidden, inter))):
                s = synth.stream_seed(seed, l, mi, synth.TAG_WEIGHT)
                t = synth.trits_torch(s, (n, k), device=DEV)
                sc = synth.ternary_scale(synth.stream_seed(seed, l, mi, synth.TAG_SCALE))
                ws.append(qmv.qmv_pack_ternary(t, sc))
                if keep_trits:
                    tl.append(t.cpu().numpy())
            norm = torch.from_numpy(
                synth.normal(synth.stream_seed(seed, l, 3, synth.TAG_MISC), (hidden,)) * 0.1 + 1.0).to(DEV)
            self.layers.append((ws[0], ws[1], ws[2], norm))
            self.trits.append(tl)
        self.arr = qmv.ffn_layer_array(self.layers)

    def h0(self, seed):
        return torch.from_numpy(synth.normal(synth.stream_seed(seed, 0, 0, synth.TAG_ACT), (self.hidden,))).to(DEV)


def chain(qmv, st, h, eps, act, record=None):
    """The launch-per-step chain; h updated in place.  record: list receiving
    each layer's intermediates (as numpy) when given."""
    H, I = st.hidden, st.inter
    x8a = torch.empty((1, H), dtype=torch.int8, device=DEV)
    sxa = torch.empty(1, dtype=torch.float32, device=DEV)
    yg = torch.empty((1, I), dtype=torch.float32, device=DEV)
    yu = torch.empty((1, I), dtype=torch.float32, device=DEV)
    ag = torch.empty((1, I), dtype=torch.int32, device=DEV)
    au = torch.empty((1, I), dtype=torch.int32, device=DEV)
    x8b = torch.empty((1, I), dtype=torch.int8, device=DEV)
    sxb = torch.empty(1, dtype=torch.float32, device=DEV)
    yd = torch.empty((1, H), dtype=torch.float32, device=DEV)
    ad = torch.empty((1, H), dtype=torch.int32, device=DEV)
    for (g, u, d, norm) in st.layers:
        h_in = h.cpu().numpy().copy() if record is not None else None
        qmv.qmv_rmsnorm_quantize(h.view(1, H), norm, eps, x8=x8a, sx=sxa)
        qmv.qmv_gemv([qmv.Problem(g, x8a, sxa, yg, ag), qmv.Problem(u, x8a, sxa, yu, au)])
        qmv.qmv_glu_quantize(yg, yu, act, x8=x8b, sx=sxb)
        qmv.qmv_gemv([qmv.Problem(d, x8b, sxb, yd, ad)])
        h.add_(yd.view(H))
        if record is not None:
            torch.cuda.synchronize()
            record.append({k_: v.cpu().numpy().copy() for k_, v in
                           dict(x8a=x8a, sxa=sxa, yg=yg, yu=yu, ag=ag, au=au, x8b=x8b, sxb=sxb, yd=yd,
                                ad=ad).items()} | {"h_in": h_in, "h_out": h.cpu().numpy().copy()})
    return h


def fused(qmv, st, h, eps, act, **kw):
    status = qmv.qmv_ffn_decode(st.arr, h, eps=eps, act=act, **kw)
    torch.cuda.synchronize()
    return int(status.cpu()[0])


CASES = [
    # hidden, inter, layers, act
    (1152, 6912, 3, 1),          # Gemma-3-1B feed-forward
    (200, 333, 4, 2),            # ragged rows and chunks, SiLU
    (1, 1, 2, 1),                # one column, one row
    (77, 5000, 2, 2),
    (2600, 700, 2, 1),           # gate/up rows of 33 chunks: loads past the register block; h beyond 2048
    (64, 96, 34, 1),             # more layers than one launch holds
]


@pytest.mark.parametrize("hidden,inter,nlayers,act", CASES)
def test_ffn_matches_chain(qmv_gpu, hidden, inter, nlayers, act):
    from ternary_matvec_amd import qmv
    say("ffn vs chain hidden=%d inter=%d layers=%d act=%d" % (hidden, inter, nlayers, act))
    st = Stack(qmv, hidden, inter, nlayers, seed=11 + hidden + inter)
    h0 = st.h0(13 + hidden)
    hc = chain(qmv, st, h0.clone(), 1e-6, act)
    hf = h0.clone()
    assert fused(qmv, st, hf, 1e-6, act) == qmv.QMV_FFN_OK
    assert torch.isfinite(hf).all()
    assert torch.equal(hf, hc), (hf - hc).abs().max().item()
    if hidden >= 64:   # (one weight per matrix may well be a zero trit)
        assert not torch.equal(hf, h0)


@pytest.mark.parametrize("hidden,inter", [(8192, 128), (64, 65536)])
def test_ffn_largest_sizes(qmv_gpu, hidden, inter):
    """The largest hidden (LDS) and inter (several gate/up tasks per workgroup)."""
    from ternary_matvec_amd import qmv
    say("ffn largest hidden=%d inter=%d" % (hidden, inter))
    st = Stack(qmv, hidden, inter, 2, seed=21)
    h0 = st.h0(23)
    hc = chain(qmv, st, h0.clone(), 1e-5, 1)
    hf = h0.clone()
    assert fused(qmv, st, hf, 1e-5, 1) == qmv.QMV_FFN_OK
    assert torch.equal(hf, hc)


def test_ffn_gemma_full_stack(qmv_gpu):
    """All 26 feed-forward layers of the Gemma-3-1B shape in one launch."""
    from ternary_matvec_amd import qmv
    say("ffn gemma 26 layers")
    st = Stack(qmv, 1152, 6912, 26, seed=31)
    h0 = st.h0(33)
    hc = chain(qmv, st, h0.clone(), 1e-6, 1)
    hf = h0.clone()
    assert fused(qmv, st, hf, 1e-6, 1) == qmv.QMV_FFN_OK
    assert torch.equal(hf, hc)
    # a second call continues from the first one's output
    hc2 = chain(qmv, st, hc.clone(), 1e-6, 1)
    assert fused(qmv, st, hf, 1e-6, 1) == qmv.QMV_FFN_OK
    assert torch.equal(hf, hc2)


def _rms_rel(k):
    return ((k + 255) // 256 + 20) * U


def _valid_rounding(x8, sx, h, rel):
    s_ref = np.maximum(np.abs(h).max(axis=1), 1e-9) / 127.0
    s = sx.astype(np.float64)
    assert np.all(np.abs(s - s_ref) <= rel * s_ref)
    q = x8.astype(np.float64)
    assert np.all(np.abs(q - h / s[:, None]) <= 0.5 + 127 * 2 * rel)
    assert np.all(np.abs(q) <= 127)


@pytest.mark.parametrize("hidden,inter,act", [(1152, 6912, 1), (200, 333, 2)])
def test_ffn_chain_against_oracle(qmv_gpu, hidden, inter, act):
    """Each layer of the chain (which the persistent launch equals bit for bit)
    against the oracle's definitions, from the layer's own input h."""
    from ternary_matvec_amd import qmv
    say("ffn chain vs oracle hidden=%d inter=%d" % (hidden, inter))
    st = Stack(qmv, hidden, inter, 2, seed=41 + hidden, keep_trits=True)
    h0 = st.h0(43)
    rec = []
    hc = chain(qmv, st, h0.clone(), 1e-6, act, record=rec)
    hf = h0.clone()
    assert fused(qmv, st, hf, 1e-6, act) == qmv.QMV_FFN_OK
    assert torch.equal(hf, hc)
    for l, r in enumerate(rec):
        g, u, d, norm = st.layers[l]
        tg, tu, td = st.trits[l]
        _valid_rounding(r["x8a"], r["sxa"], oracle.rmsnorm(r["h_in"][None, :], norm.cpu().numpy(), 1e-6),
                        _rms_rel(hidden))
        assert np.array_equal(r["ag"], oracle.matmul_int(r["x8a"], tg))
        assert np.array_equal(r["au"], oracle.matmul_int(r["x8a"], tu))
        for y, a, w in ((r["yg"], r["ag"], g), (r["yu"], r["au"], u)):
            ref = oracle.dequant(a, r["sxa"], float(w.scale.cpu()[0])).astype(np.float64)
            assert np.all(np.abs(y - ref) <= 3 * U * np.abs(ref))
        _valid_rounding(r["x8b"], r["sxb"], oracle.glu(r["yg"], r["yu"], act), 4e-7)
        assert np.array_equal(r["ad"], oracle.matmul_int(r["x8b"], td))
        ref = oracle.dequant(r["ad"], r["sxb"], float(d.scale.cpu()[0])).astype(np.float64)
        assert np.all(np.abs(r["yd"] - ref) <= 3 * U * np.abs(ref))
        assert np.array_equal(r["h_out"], (r["h_in"] + r["yd"][0]).astype(np.float32))


def test_ffn_cancel_and_timeout_leave_a_clean_workspace(qmv_gpu):
    from ternary_matvec_amd import qmv
    say("ffn cancel / timeout")
    st = Stack(qmv, 300, 900, 3, seed=51)
    h0 = st.h0(53)
    hc = chain(qmv, st, h0.clone(), 1e-6, 2)
    ws = qmv.ffn_workspace(300, 900, torch.device(DEV))
    # a cancel word already set: every launch stops at its first wait, h untouched
    dev_word = torch.ones(1, dtype=torch.int32, device=DEV)
    host_word = torch.ones(1, dtype=torch.int32).pin_memory()
    for word in (dev_word, host_word):
        h = h0.clone()
        assert fused(qmv, st, h, 1e-6, 2, workspace=ws, cancel=word) == qmv.QMV_FFN_CANCELLED
        assert torch.equal(h, h0)
        h = h0.clone()
        assert fused(qmv, st, h, 1e-6, 2, workspace=ws) == qmv.QMV_FFN_OK
        assert torch.equal(h, hc)
    # a cleared word does not stop it
    host_word.zero_()
    h = h0.clone()
    assert fused(qmv, st, h, 1e-6, 2, workspace=ws, cancel=host_word) == qmv.QMV_FFN_OK
    assert torch.equal(h, hc)
    # one poll per wait: done or timed out, never a hang; then exact again
    h = h0.clone()
    s1 = fused(qmv, st, h, 1e-6, 2, workspace=ws, spin_limit=1)
    assert s1 in (qmv.QMV_FFN_OK, qmv.QMV_FFN_TIMEOUT)
    if s1 == qmv.QMV_FFN_OK:
        assert torch.equal(h, hc)
    # the status word's old value is ignored; the sync words are zero again
    status = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    h = h0.clone()
    assert fused(qmv, st, h, 1e-6, 2, workspace=ws, status=status) == qmv.QMV_FFN_OK
    assert torch.equal(h, hc)
    # the exit counters and the two accumulators (the workspace's last bytes) are zero again
    assert int(ws[512:2564].count_nonzero()) == 0
    assert int(ws[-2 * 4 * 320:].count_nonzero()) == 0


def test_ffn_error_stops_later_launches(qmv_gpu):
    """With more layers than one launch holds, a cancelled first launch makes the
    later launches of the call do nothing."""
    from ternary_matvec_amd import qmv
    say("ffn cancel across launches")
    st = Stack(qmv, 64, 96, 40, seed=61)
    h0 = st.h0(63)
    word = torch.ones(1, dtype=torch.int32, device=DEV)
    h = h0.clone()
    assert fused(qmv, st, h, 1e-6, 1, cancel=word) == qmv.QMV_FFN_CANCELLED
    assert torch.equal(h, h0)


def test_ffn_trace(qmv_gpu):
    """Stamps in order within every workgroup, and no gate/up task starts a layer
    before every down task of the previous layer has acknowledged its adds."""
    from ternary_matvec_amd import qmv
    say("ffn trace")
    H, I, L = 1152, 6912, 4
    S = qmv.QMV_FFN_TRACE_STAMPS
    st = Stack(qmv, H, I, L, seed=71)
    grid = qmv.qmv_ffn_grid()
    assert grid >= 1
    trace = torch.zeros((grid, 1 + S * L), dtype=torch.int64, device=DEV)
    h = st.h0(73)
    hc = chain(qmv, st, h.clone(), 1e-6, 1)
    assert fused(qmv, st, h, 1e-6, 1, trace=trace) == qmv.QMV_FFN_OK
    assert torch.equal(h, hc)
    t = trace.cpu().numpy()
    gu_tasks = (I + 31) // 32
    gu = t[:min(grid, gu_tasks)]
    assert np.all(t[:, 0] > 0)
    times = t[:, 1:].reshape(grid, L, S)[:, :, :S - 1]          # slot S-1 counts poll rounds
    for row in np.concatenate([t[:, :1], times.reshape(grid, -1)], axis=1):
        nz = row[row > 0]
        assert np.all(np.diff(nz) >= 0)
    st_gu = gu[:, 1:].reshape(len(gu), L, S)
    assert np.all(st_gu[:, :, :6] > 0)
    dn = t[:, 1:].reshape(grid, L, S)
    dn = dn[dn[:, 0, 9] > 0]                        # workgroups with a down task
    assert len(dn) > 0
    for l in range(1, L):
        assert st_gu[:, l, 1].min() >= dn[:, l - 1, 9].max()


def test_ffn_graph_replay(qmv_gpu):
    from ternary_matvec_amd import qmv
    say("ffn graph replay")
    st = Stack(qmv, 1152, 6912, 2, seed=81)
    h0 = st.h0(83)
    ref = h0.clone()
    ws = qmv.ffn_workspace(1152, 6912, torch.device(DEV))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    assert fused(qmv, st, ref, 1e-6, 1, workspace=ws, status=status) == qmv.QMV_FFN_OK
    h = torch.empty_like(h0)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            h.copy_(h0)
            qmv.qmv_ffn_decode(st.arr, h, eps=1e-6, act=1, workspace=ws, status=status, stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for _ in range(3):
        h.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(status.cpu()[0]) == qmv.QMV_FFN_OK
        assert torch.equal(h, ref)
