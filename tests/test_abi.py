"""The C-ABI library loads and exports every symbol include/qmv.h declares.

CPU only: these calls validate host-side arguments and return before any
device work, so no GPU is needed.
"""
import ctypes
import os
import re

import pytest

from ternary_matvec_amd import qmv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "qmv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qmv.LIB_PATH):
        pytest.fail("libqmv.so is not built (run __graft_entry__.build())")
    return qmv.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert "qmv_gemv" in names and "qmv_lmhead_argmax" in names
    for name in names:
        assert hasattr(lib, name), name
    # the binding declares exactly the header's functions
    assert sorted(qmv.SIGNATURES) == names


def test_core_entry_points_present(lib):
    for name in ("qmv_pack_ternary", "qmv_pack_int8", "qmv_quantize_act", "qmv_gemv", "qmv_gemm_prefill",
                 "qmv_lmhead_argmax"):
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert "gfx950" in qmv.version()
    assert qmv.status_str(0) == "ok"
    assert qmv.status_str(qmv.QMV_EWORKSPACE) == "workspace missing or too small"
    assert qmv.status_str(12345) == "unknown status"


def test_packed_bytes(lib):
    assert qmv.qmv_packed_bytes(qmv.QMV_W_TERNARY5, 1024, 1152) == 1024 * 240
    assert qmv.qmv_packed_bytes(qmv.QMV_W_TERNARY5, 1152, 6912) == 1152 * 1392
    assert qmv.qmv_packed_bytes(qmv.QMV_W_TERNARY5, 3, 81) == 3 * 32
    assert qmv.qmv_packed_bytes(qmv.QMV_W_INT8, 768, 288) == 768 * 288
    assert qmv.qmv_packed_bytes(qmv.QMV_W_INT8, 2, 17) == 64
    assert qmv.qmv_packed_bytes(qmv.QMV_W_INT8_G128, 6912, 1152) == 6912 * 1152
    assert qmv.qmv_packed_bytes(qmv.QMV_W_INT8_G128, 3, 300) == 3 * 304
    assert qmv.qmv_packed_bytes(7, 2, 17) == -1
    assert qmv.qmv_packed_bytes(qmv.QMV_W_TERNARY5, 0, 17) == -1


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_host_validation_errors(lib):
    desc = qmv.qmv_weight()
    s = None
    # null pointers
    assert lib.qmv_pack_ternary(None, 4, 4, 1.0, _fake(4096), _fake(8192), None, ctypes.byref(desc), s) == qmv.QMV_EINVAL
    assert lib.qmv_quantize_act(None, 1, 4, _fake(4096), _fake(8192), s) == qmv.QMV_EINVAL
    # bad shapes
    assert lib.qmv_pack_ternary(_fake(64), 0, 4, 1.0, _fake(4096), _fake(8192), None, None, s) == qmv.QMV_ESHAPE
    assert lib.qmv_quantize_act(_fake(64), 1, 0, _fake(4096), _fake(8192), s) == qmv.QMV_ESHAPE
    # misaligned packed buffer, non-finite scale
    assert lib.qmv_pack_ternary(_fake(64), 2, 4, 1.0, _fake(4097), _fake(8192), None, None, s) == qmv.QMV_EINVAL
    assert lib.qmv_pack_ternary(_fake(64), 2, 4, float("inf"), _fake(4096), _fake(8192), None, None, s) == qmv.QMV_EVALUE
    # int8 K limit keeps every dot inside int32
    assert lib.qmv_pack_int8(_fake(64), 2, 70000, _fake(4096), _fake(8192), None, s) == qmv.QMV_ESHAPE
    # several activation sets in one launch
    acts = (qmv.qmv_act * 9)()
    for i in range(9):
        acts[i] = qmv.qmv_act(4096, 2, 64, 8192, 12288)
    assert lib.qmv_quantize_act_many(None, 1, s) == qmv.QMV_EINVAL
    assert lib.qmv_quantize_act_many(acts, 0, s) == qmv.QMV_ESHAPE
    assert lib.qmv_quantize_act_many(acts, 9, s) == qmv.QMV_ESHAPE
    acts[1].sx = None
    assert lib.qmv_quantize_act_many(acts, 2, s) == qmv.QMV_EINVAL
    acts[1].sx, acts[1].k = 12288, 0
    assert lib.qmv_quantize_act_many(acts, 2, s) == qmv.QMV_ESHAPE
    acts[1].k, acts[1].m = 64, 1 << 31
    assert lib.qmv_quantize_act_many(acts, 2, s) == qmv.QMV_ESHAPE
    # group-scaled int8: nulls, shapes, alignment
    assert lib.qmv_pack_int8_grouped(_fake(64), 2, 300, _fake(4096), None, None, s) == qmv.QMV_EINVAL
    assert lib.qmv_pack_int8_grouped(_fake(64), 2, 70000, _fake(4096), _fake(8192), None, s) == qmv.QMV_ESHAPE
    assert lib.qmv_pack_int8_grouped(_fake(64), (1 << 20) + 1, 64, _fake(4096), _fake(8192), None, s) == \
        qmv.QMV_ESHAPE
    assert lib.qmv_pack_int8_grouped(_fake(64), 1 << 20, 4096, _fake(4096), _fake(8192), None, s) == qmv.QMV_ESHAPE
    assert lib.qmv_pack_int8_grouped(_fake(64), 2, 300, _fake(4100), _fake(8192), None, s) == qmv.QMV_EINVAL
    assert lib.qmv_quantize_act_grouped(_fake(64), 1, 0, _fake(4096), _fake(8192), s) == qmv.QMV_ESHAPE
    assert lib.qmv_quantize_act_grouped(None, 1, 4, _fake(4096), _fake(8192), s) == qmv.QMV_EINVAL
    # lm_head
    assert lib.qmv_lmhead_argmax(_fake(4096), _fake(64), 10, 8, None, None, None, _fake(256), 4096, s) == qmv.QMV_EINVAL
    assert lib.qmv_lmhead_argmax(_fake(4096), _fake(64), 10, 8, _fake(64), None, None, None, 0, s) == qmv.QMV_EWORKSPACE
    assert qmv.qmv_lmhead_workspace_bytes(262144, 1152) > 0
    # fused RMSNorm / gate quantisation
    assert lib.qmv_rmsnorm_quantize(_fake(64), None, 1, 4, 1e-5, _fake(4096), _fake(8192), s) == qmv.QMV_EINVAL
    assert lib.qmv_rmsnorm_quantize(_fake(64), _fake(64), 1, 0, 1e-5, _fake(4096), _fake(8192), s) == qmv.QMV_ESHAPE
    assert lib.qmv_rmsnorm_quantize(_fake(64), _fake(64), 1, 4, -1.0, _fake(4096), _fake(8192), s) == qmv.QMV_EVALUE
    assert lib.qmv_rmsnorm_quantize(_fake(64), _fake(64), 1, 4, float("nan"), _fake(4096), _fake(8192), s) == \
        qmv.QMV_EVALUE
    assert lib.qmv_glu_quantize(_fake(64), _fake(64), 1, 4, 3, _fake(4096), _fake(8192), s) == qmv.QMV_EINVAL
    assert lib.qmv_glu_quantize(_fake(64), None, 1, 4, 1, _fake(4096), _fake(8192), s) == qmv.QMV_EINVAL
    assert lib.qmv_glu_quantize(_fake(64), _fake(64), 0, 4, 1, _fake(4096), _fake(8192), s) == qmv.QMV_ESHAPE
    # sketch head: shape limits, alignment, workspace
    assert qmv.qmv_sketch_bytes(262144, 1152) > 0 and qmv.qmv_sketch_workspace_bytes(262144, 1152) > 0
    for v, k in [(0, 64), (10, 7), (10, 12), (10, 8200), (10, 0)]:
        assert qmv.qmv_sketch_bytes(v, k) == -1
    assert lib.qmv_sketch_build(_fake(4096), 10, 64, _fake(4097), 1 << 20, s) == qmv.QMV_EINVAL
    assert lib.qmv_sketch_build(_fake(4096), 10, 60, _fake(4096), 1 << 20, s) == qmv.QMV_ESHAPE
    assert lib.qmv_sketch_build(_fake(4096), 10, 64, _fake(4096), 16, s) == qmv.QMV_EWORKSPACE
    assert lib.qmv_lmhead_sketch_argmax(_fake(4096), _fake(4096), _fake(64), 10, 64, None, None, None, None,
                                        _fake(4096), 1 << 20, s) == qmv.QMV_EINVAL
    assert lib.qmv_lmhead_sketch_argmax(_fake(4096), _fake(4096), _fake(64), 10, 64, _fake(64), None, None, None,
                                        _fake(4096), 16, s) == qmv.QMV_EWORKSPACE
    assert lib.qmv_lmhead_sketch_argmax(_fake(4096), _fake(4096), _fake(68), 10, 64, _fake(64), None, None, None,
                                        _fake(4096), 1 << 20, s) == qmv.QMV_EINVAL   # x not 16-byte aligned


def _problem(wtype=qmv.QMV_W_TERNARY5, n=64, k=80, m=1, data=4096):
    p = qmv.qmv_problem()
    p.w.wtype, p.w.reserved, p.w.n, p.w.k, p.w.data, p.w.scale = wtype, 0, n, k, data, 8192
    p.x8, p.sx, p.m, p.y, p.acc = 12288, 16384, m, 20480, None
    return p


def test_gemv_validation(lib):
    arr = (qmv.qmv_problem * 2)(_problem(), _problem(n=100, k=1152, m=3))
    need = lib.qmv_gemv_workspace_bytes(arr, 2)
    assert need > 0 and need % 256 == 0
    assert lib.qmv_workspace_bytes(arr, 2) >= need
    # workspace missing / too small / misaligned
    assert lib.qmv_gemv(arr, 2, None, 0, None) == qmv.QMV_EWORKSPACE
    assert lib.qmv_gemv(arr, 2, _fake(1 << 20), need - 1, None) == qmv.QMV_EWORKSPACE
    assert lib.qmv_gemv(arr, 2, _fake((1 << 20) + 64), need, None) == qmv.QMV_EWORKSPACE
    # m out of range for the GEMV
    bad = (qmv.qmv_problem * 1)(_problem(m=17))
    assert lib.qmv_gemv(bad, 1, _fake(1 << 20), 1 << 20, None) == qmv.QMV_ESHAPE
    assert lib.qmv_gemv_workspace_bytes(bad, 1) == -1
    assert lib.qmv_workspace_bytes(bad, 1) == lib.qmv_prefill_workspace_bytes(bad, 1) > 0
    # unknown weight type, reserved field, misaligned weights, null y
    bad = (qmv.qmv_problem * 1)(_problem(wtype=9))
    assert lib.qmv_gemv(bad, 1, _fake(1 << 20), 1 << 20, None) == qmv.QMV_EUNSUPPORTED
    assert lib.qmv_workspace_bytes(bad, 1) == -1
    p = _problem()
    p.w.reserved = 1
    assert lib.qmv_gemv((qmv.qmv_problem * 1)(p), 1, _fake(1 << 20), 1 << 20, None) == qmv.QMV_EINVAL
    p = _problem(data=4100)
    assert lib.qmv_gemv((qmv.qmv_problem * 1)(p), 1, _fake(1 << 20), 1 << 20, None) == qmv.QMV_EINVAL
    p = _problem()
    p.y = None
    assert lib.qmv_gemv((qmv.qmv_problem * 1)(p), 1, _fake(1 << 20), 1 << 20, None) == qmv.QMV_EINVAL
    # activations too large to stage for 16 tokens
    big = (qmv.qmv_problem * 1)(_problem(n=64, k=1 << 20, m=16))
    assert lib.qmv_gemv(big, 1, _fake(1 << 20), 1 << 30, None) == qmv.QMV_ESHAPE
    # count
    assert lib.qmv_gemv(arr, 0, _fake(1 << 20), need, None) == qmv.QMV_ESHAPE
    assert lib.qmv_gemv(None, 1, _fake(1 << 20), need, None) == qmv.QMV_EINVAL


def test_plan_validation(lib):
    import torch
    arr = (qmv.qmv_problem * 2)(_problem(), _problem(n=100, k=1152, m=3))
    h = ctypes.c_void_p()
    assert lib.qmv_plan_create(5, arr, 2, ctypes.byref(h)) == qmv.QMV_EINVAL
    assert lib.qmv_plan_create(qmv.QMV_PLAN_GEMV, arr, 2, None) == qmv.QMV_EINVAL
    assert lib.qmv_plan_create(qmv.QMV_PLAN_GEMV, arr, 0, ctypes.byref(h)) == qmv.QMV_ESHAPE
    bad = (qmv.qmv_problem * 1)(_problem(m=17))
    assert lib.qmv_plan_create(qmv.QMV_PLAN_GEMV, bad, 1, ctypes.byref(h)) == qmv.QMV_ESHAPE and not h.value
    g = (qmv.qmv_problem * 1)(_problem(wtype=qmv.QMV_W_INT8_G128))
    assert lib.qmv_plan_create(qmv.QMV_PLAN_PREFILL, g, 1, ctypes.byref(h)) == qmv.QMV_EUNSUPPORTED
    assert lib.qmv_plan_workspace_bytes(None) == -1
    assert lib.qmv_plan_upload(None, _fake(1 << 20), 1 << 20, None) == qmv.QMV_EINVAL
    assert lib.qmv_plan_launch(None, _fake(1 << 20), 1 << 20, None) == qmv.QMV_EINVAL
    lib.qmv_plan_destroy(None)
    for kind in (qmv.QMV_PLAN_GEMV, qmv.QMV_PLAN_PREFILL, qmv.QMV_PLAN_GEMV_DOT, qmv.QMV_PLAN_GEMV_SKIP_ZERO):
        assert lib.qmv_plan_create(kind, arr, 2, ctypes.byref(h)) == qmv.QMV_OK and h.value
        need = lib.qmv_plan_workspace_bytes(h)
        assert need > 0
        assert need <= (lib.qmv_gemv_workspace_bytes if kind != qmv.QMV_PLAN_PREFILL
                        else lib.qmv_prefill_workspace_bytes)(arr, 2)
        assert lib.qmv_plan_launch(h, None, 0, None) == qmv.QMV_EWORKSPACE
        assert lib.qmv_plan_upload(h, _fake(1 << 20), need - 1, None) == qmv.QMV_EWORKSPACE
        assert lib.qmv_plan_launch(h, _fake((1 << 20) + 16), need, None) == qmv.QMV_EWORKSPACE
        if not torch.cuda.is_available():      # a plan made with no usable device cannot run
            assert lib.qmv_plan_launch(h, _fake(1 << 20), need, None) == qmv.QMV_EHIP
        lib.qmv_plan_destroy(h)


def test_lmhead_static_validation(lib):
    s = None
    assert lib.qmv_lmhead_argmax_static(_fake(4096), _fake(64), 10, 8, None, None, None, s) == qmv.QMV_EINVAL
    assert lib.qmv_lmhead_argmax_static(None, _fake(64), 10, 8, _fake(64), None, None, s) == qmv.QMV_EINVAL
    assert lib.qmv_lmhead_argmax_static(_fake(4096), _fake(64), 0, 8, _fake(64), None, None, s) == qmv.QMV_ESHAPE
    # the static scratch holds the maxima of at most 2^21 rows
    assert lib.qmv_lmhead_argmax_static(_fake(4096), _fake(64), (1 << 21) + 64, 8, _fake(64), None, None, s) == \
        qmv.QMV_ESHAPE


def test_read_probe_rejects_bad_arguments(lib):
    """qmv_read_probe validates on the host: null pointers, misaligned or ragged sizes."""
    import ctypes
    EINVAL = -1
    out = ctypes.c_uint32(0)
    assert lib.qmv_read_probe(None, 16, ctypes.addressof(out), None) == EINVAL
    assert lib.qmv_read_probe(ctypes.c_void_p(16), 16, None, None) == EINVAL
    assert lib.qmv_read_probe(ctypes.c_void_p(16), 15, ctypes.addressof(out), None) == EINVAL
    assert lib.qmv_read_probe(ctypes.c_void_p(17), 16, ctypes.addressof(out), None) == EINVAL
    assert lib.qmv_read_probe(ctypes.c_void_p(16), -16, ctypes.addressof(out), None) == EINVAL
    assert lib.qmv_read_probe(ctypes.c_void_p(16), 0, ctypes.addressof(out), None) == 0


def test_gemv_grouped_validation(lib):
    g = qmv.QMV_W_INT8_G128
    arr = (qmv.qmv_problem * 3)(_problem(wtype=g, n=6912, k=1152), _problem(n=100, k=1152, m=3),
                                _problem(wtype=g, n=1152, k=6912, m=16))
    need = lib.qmv_gemv_workspace_bytes(arr, 3)
    assert need > 0 and need % 256 == 0
    # the grouped path has no single exact dot: acc must be NULL
    p = _problem(wtype=g)
    p.acc = 24576
    assert lib.qmv_gemv((qmv.qmv_problem * 1)(p), 1, _fake(1 << 20), 1 << 20, None) == qmv.QMV_EINVAL
    # staged activations past the LDS: 16 tokens x 16384 columns
    big = (qmv.qmv_problem * 1)(_problem(wtype=g, n=64, k=16384, m=16))
    assert lib.qmv_gemv_workspace_bytes(big, 1) == -1
    assert lib.qmv_gemv(big, 1, _fake(1 << 20), 1 << 30, None) == qmv.QMV_ESHAPE
    # rows past the tile-entry limit
    big = (qmv.qmv_problem * 1)(_problem(wtype=g, n=(1 << 20) + 1, k=64))
    assert lib.qmv_gemv_workspace_bytes(big, 1) == -1
    # prefill takes ternary weights only
    assert lib.qmv_prefill_workspace_bytes((qmv.qmv_problem * 1)(_problem(wtype=g)), 1) == -1


def _ffn_layers(n, hidden=1152, inter=6912):
    arr = (qmv.qmv_ffn_layer * n)()
    for i in range(n):
        for name, (rows, cols) in (("gate", (inter, hidden)), ("up", (inter, hidden)), ("down", (hidden, inter))):
            w = getattr(arr[i], name)
            w.wtype, w.n, w.k, w.data, w.scale = qmv.QMV_W_TERNARY5, rows, cols, 4096 * (i + 1), 64
        arr[i].norm = 128
    return arr


def test_ffn_workspace_bytes(lib):
    # control words; 8 replicas (4 KiB-rounded) of a tag per down task (at most one per 8
    # chunks of a 64-row group) and of two parities of the GLU maxima of the 32-row gate/up
    # tasks (8-byte records, an even count); inter 8-byte GLU records (256-byte rounded); two
    # int32 accumulators of round_up(hidden, 64)
    assert qmv.qmv_ffn_workspace_bytes(1152, 6912) == 4096 + 8 * 4096 + 8 * 4096 + 8 * 6912 + 2 * 4 * 1152
    assert qmv.qmv_ffn_workspace_bytes(5, 3) == 4096 + 8 * 4096 + 8 * 4096 + 256 + 2 * 4 * 64
    assert qmv.qmv_ffn_workspace_bytes(0, 8) == -1
    assert qmv.qmv_ffn_workspace_bytes(8, 0) == -1
    assert qmv.qmv_ffn_workspace_bytes(qmv.QMV_FFN_MAX_HIDDEN + 1, 8) == -1
    assert qmv.qmv_ffn_workspace_bytes(8, qmv.QMV_FFN_MAX_INTER + 1) == -1


def test_ffn_decode_validation(lib):
    """qmv_ffn_decode refuses bad arguments on the host, before any device work."""
    ws_need = qmv.qmv_ffn_workspace_bytes(1152, 6912)
    ws, st, h, s = _fake(1 << 20), _fake(64), _fake(8192), None

    def call(arr, n=None, h_=h, eps=1e-6, act=qmv.QMV_ACT_GELU_TANH, ws_=ws, wsb=ws_need, spin=0, st_=st,
             trace=None):
        return lib.qmv_ffn_decode(arr, len(arr) if n is None else n, h_, ctypes.c_float(eps), act, ws_, wsb, None,
                                  spin, st_, trace, s)

    arr = _ffn_layers(3)
    assert lib.qmv_ffn_decode(None, 3, h, ctypes.c_float(1e-6), 1, ws, ws_need, None, 0, st, None, s) == \
        qmv.QMV_EINVAL
    assert call(arr, h_=None) == qmv.QMV_EINVAL
    assert call(arr, st_=None) == qmv.QMV_EINVAL                 # the status word is required
    assert call(arr, n=0) == qmv.QMV_ESHAPE
    assert call(arr, eps=-1.0) == qmv.QMV_EVALUE
    assert call(arr, eps=float("inf")) == qmv.QMV_EVALUE
    assert call(arr, act=3) == qmv.QMV_EINVAL
    assert call(arr, spin=-1) == qmv.QMV_EVALUE
    assert call(arr, ws_=None) == qmv.QMV_EWORKSPACE
    assert call(arr, ws_=_fake((1 << 20) + 16)) == qmv.QMV_EWORKSPACE   # not 256-byte aligned
    assert call(arr, wsb=ws_need - 1) == qmv.QMV_EWORKSPACE
    # a trace covers one launch
    assert call(_ffn_layers(qmv.QMV_FFN_LAUNCH_LAYERS + 1), trace=_fake(64)) == qmv.QMV_EINVAL
    # shapes: every layer the same hidden / inter, down the transpose of gate / up
    bad = _ffn_layers(2)
    bad[1].up.n = 6911
    assert call(bad) == qmv.QMV_ESHAPE
    bad = _ffn_layers(2)
    bad[0].down.k = 1152
    assert call(bad) == qmv.QMV_ESHAPE
    assert call(_ffn_layers(1, hidden=qmv.QMV_FFN_MAX_HIDDEN + 1, inter=64)) == qmv.QMV_ESHAPE
    assert call(_ffn_layers(1, hidden=64, inter=qmv.QMV_FFN_MAX_INTER + 1)) == qmv.QMV_ESHAPE
    # ternary weights only, aligned, with scales and RMSNorm weights
    bad = _ffn_layers(2)
    bad[1].down.wtype = qmv.QMV_W_INT8
    assert call(bad) == qmv.QMV_EUNSUPPORTED
    bad = _ffn_layers(2)
    bad[0].gate.data = 4096 + 8
    assert call(bad) == qmv.QMV_EINVAL
    bad = _ffn_layers(2)
    bad[0].up.scale = None
    assert call(bad) == qmv.QMV_EINVAL
    bad = _ffn_layers(2)
    bad[1].norm = None
    assert call(bad) == qmv.QMV_EINVAL
    import torch
    if not torch.cuda.is_available():   # valid arguments and no usable device
        assert call(arr) == qmv.QMV_EHIP
        g = ctypes.c_int32(0)
        assert lib.qmv_ffn_grid(ctypes.byref(g)) == qmv.QMV_EHIP
    assert lib.qmv_ffn_grid(None) == qmv.QMV_EINVAL


def test_mfma_probe_validation(lib):
    ops = ctypes.c_int64(0)
    out = _fake(64)
    assert lib.qmv_mfma_probe(0, 10, None, ctypes.byref(ops), None) == qmv.QMV_EINVAL
    assert lib.qmv_mfma_probe(0, 10, out, None, None) == qmv.QMV_EINVAL
    assert lib.qmv_mfma_probe(2, 10, out, ctypes.byref(ops), None) == qmv.QMV_EINVAL
    assert lib.qmv_mfma_probe(1, 0, out, ctypes.byref(ops), None) == qmv.QMV_EINVAL
    assert lib.qmv_mfma_probe(1, (1 << 20) + 1, out, ctypes.byref(ops), None) == qmv.QMV_EINVAL
