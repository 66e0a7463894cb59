"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The benchmark's own stacks are built (bench.DecodeStack / bench.PrefillStack:
the same grouped problem lists and plan launches), one pass
is run, and the results are checked against the CPU oracle:
  * activations: every int8 code and scale, bit-exact;
  * packed weights: every byte, through the oracle's unpacker, against the
    trits regenerated from their counter-based streams;
  * outputs: sampled rows of every matrix (first, last and random rows; all
    tokens), y within 1e-6 relative of the oracle's exact dequantised value and
    exactly 0 where the integer dot is 0;
  * the output layer: all 262144 logits and the greedy index.
"""
import sys

import numpy as np
import pytest
import torch

import bench
import oracle
from ternary_matvec_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SAMPLE_ROWS = 24


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _sample_rows(n, seed):
    rng = np.random.default_rng(seed)
    rows = {0, n - 1} | set(int(r) for r in rng.integers(0, n, SAMPLE_ROWS))
    return np.array(sorted(rows))


def _trit_rows(seed, k, rows):
    return np.stack([synth.trits(seed, (1, k), start=int(r) * k)[0] for r in rows])


def _check_y(y, acc_ref, sx, sw):
    y_ref = oracle.dequant(acc_ref, sx, sw)
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    tol = 1e-6 * np.abs(y_ref.astype(np.float64))
    assert np.all(err <= tol), float((err - tol).max())
    assert np.all(y[acc_ref == 0] == 0.0)


def _check_stack_outputs(st, x8_by_k, sx_by_k, y_of, config_id, tokens):
    """Sampled rows of every matrix against the oracle.  x8_by_k / sx_by_k are the
    oracle's own quantisations (already checked equal to the GPU's)."""
    for i, (layer, mid, name, n, k, slot) in enumerate(st.specs):
        rows = _sample_rows(n, 1000 * layer + mid)
        t = _trit_rows(synth.stream_seed(config_id, layer, mid, synth.TAG_WEIGHT), k, rows)
        q = x8_by_k[k][slot * tokens:(slot + 1) * tokens]
        sx = sx_by_k[k][slot * tokens:(slot + 1) * tokens]
        sw = st.scales[i:i + 1].cpu().numpy()[0]
        assert sw == np.float32(synth.ternary_scale(synth.stream_seed(config_id, layer, mid, synth.TAG_SCALE)))
        acc_ref = oracle.matmul_int(q, t)
        _check_y(y_of(i)[:, rows], acc_ref, sx, sw)


def _check_packed(st, config_id):
    """Every packed byte of every matrix: the oracle unpacks the GPU's buffer and
    the result must equal the regenerated trits (and hold no byte >= 243)."""
    pool = st.pool[0].cpu().numpy()
    off = 0
    from ternary_matvec_amd import qmv
    for (layer, mid, name, n, k, slot) in st.specs:
        nb = qmv.qmv_packed_bytes(qmv.QMV_W_TERNARY5, n, k)
        t_gpu, invalid = oracle.unpack_trit5(pool[off:off + nb], n, k)
        assert invalid == 0
        rows = _sample_rows(n, 7 + 1000 * layer + mid)
        np.testing.assert_array_equal(
            t_gpu[rows], _trit_rows(synth.stream_seed(config_id, layer, mid, synth.TAG_WEIGHT), k, rows))
        # the full matrix: regenerate it on the device (bit-identical integer draws)
        t_all = synth.trits_torch(synth.stream_seed(config_id, layer, mid, synth.TAG_WEIGHT), (n, k), device=DEV)
        np.testing.assert_array_equal(t_gpu, t_all.cpu().numpy())
        off += nb


def _run_decode_step(st, stream):
    from ternary_matvec_amd import qmv
    qmv.qmv_quantize_act_many(st.acts, stream=stream)   # the bench's one launch for both widths
    st.plans[0].launch(stream)
    torch.cuda.synchronize()


def _oracle_quant(st):
    x8, sx = {}, {}
    for k in st.x:
        q_ref, s_ref = oracle.quantize_rows(st.x_host[k])
        np.testing.assert_array_equal(st.x8[k].cpu().numpy(), q_ref)
        np.testing.assert_array_equal(st.sx[k].cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
        x8[k], sx[k] = q_ref, s_ref
    return x8, sx


@pytest.fixture(scope="module")
def gemma_stack(qmv_gpu):
    say("building the Gemma-3-1B x26 decode stack (one copy)")
    st = bench.DecodeStack(synth.GEMMA_MATS, synth.GEMMA_LAYERS, synth.CONFIG_GEMMA_DECODE, 1, 1,
                           torch.device(DEV))
    yield st
    del st
    torch.cuda.empty_cache()


def test_fullsize_gemma_decode_step(gemma_stack):
    st = gemma_stack
    say("gemma decode step: 156 matrices, one grouped launch")
    stream = torch.cuda.current_stream()
    for y in st.y.values():
        y.fill_(float("nan"))
    _run_decode_step(st, stream)
    x8, sx = _oracle_quant(st)
    _check_stack_outputs(st, x8, sx, lambda i: st.y[i].cpu().numpy(), synth.CONFIG_GEMMA_DECODE, 1)
    # a second step over the same buffers gives the same bits
    first = {i: y.clone() for i, y in st.y.items()}
    _run_decode_step(st, stream)
    for i, y in st.y.items():
        assert torch.equal(y, first[i])


def test_fullsize_gemma_packed_bytes(gemma_stack):
    say("gemma packed bytes: 156 matrices through the oracle's unpacker")
    _check_packed(gemma_stack, synth.CONFIG_GEMMA_DECODE)


def test_fullsize_gemma_prefill_512(gemma_stack):
    from ternary_matvec_amd import qmv
    st = gemma_stack
    say("gemma prefill: 512 tokens x 156 matrices, one launch")
    ps = bench.PrefillStack(st, 512, torch.device(DEV))
    stream = torch.cuda.current_stream()
    for y in ps.y.values():
        y.fill_(float("nan"))
    qmv.qmv_quantize_act_many(ps.acts, stream=stream)
    ps.plan.launch(stream)
    torch.cuda.synchronize()
    x8, sx = {}, {}
    for k in ps.x:
        q_ref, s_ref = oracle.quantize_rows(ps.x[k].cpu().numpy())
        np.testing.assert_array_equal(ps.x8[k].cpu().numpy(), q_ref)
        np.testing.assert_array_equal(ps.sx[k].cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
        x8[k], sx[k] = q_ref, s_ref
    for i, y in ps.y.items():
        assert not torch.isnan(y).any(), "prefill output %d has elements never written" % i
    _check_stack_outputs(st, x8, sx, lambda i: ps.y[i].cpu().numpy(), synth.CONFIG_GEMMA_DECODE, 512)
    del ps
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [1, 4, 16])
def test_fullsize_bitnet_decode(qmv_gpu, m):
    say("bitnet-large x24 decode, %d tokens" % m)
    st = bench.DecodeStack(synth.BITNET_MATS, synth.BITNET_LAYERS, synth.CONFIG_BITNET, m, 1, torch.device(DEV))
    for y in st.y.values():
        y.fill_(float("nan"))
    _run_decode_step(st, torch.cuda.current_stream())
    x8, sx = _oracle_quant(st)
    _check_stack_outputs(st, x8, sx, lambda i: st.y[i].cpu().numpy(), synth.CONFIG_BITNET, m)
    del st
    torch.cuda.empty_cache()


def test_fullsize_output_layer(qmv_gpu):
    from ternary_matvec_amd import qmv
    say("output layer 262144 x 1152 bf16 + greedy argmax")
    v, k = synth.HEAD_V, synth.HEAD_K
    w0 = synth.normal_torch(synth.stream_seed(synth.CONFIG_HEAD, 0, 0, synth.TAG_HEAD), (v, k), std=0.02, device=DEV)
    w = w0.to(torch.bfloat16)
    del w0
    x = synth.normal(synth.stream_seed(synth.CONFIG_HEAD, 0, 0, synth.TAG_ACT), (k,))
    idx, mx, logits = qmv.qmv_lmhead_argmax(w, torch.from_numpy(x).to(DEV), want_logits=True)
    torch.cuda.synchronize()
    w_bits = w.view(torch.int16).cpu().numpy().view(np.uint16)
    ref, ref_idx = oracle.lmhead(w_bits, x)
    wf = synth.bf16_bits_to_f32(w_bits).astype(np.float64)
    gamma = k * 2.0 ** -24 / (1 - k * 2.0 ** -24)
    tol = np.maximum(2e-2 * np.abs(ref), gamma * (np.abs(wf) @ np.abs(x.astype(np.float64))))
    lg = logits.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(lg - ref) <= tol), float((np.abs(lg - ref) - tol).max())
    i = int(idx.item())
    if i != ref_idx:
        assert abs(ref[i] - ref[ref_idx]) <= max(tol[i], tol[ref_idx]), (i, ref_idx)
    assert mx.item() == logits[i].item()
