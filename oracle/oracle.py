"""NumPy-facing wrappers around the C oracle (oracle/qmv_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark; never by the product library.  Each wrapper only
marshals arrays; all arithmetic is in the C file, which cites the passages of
the source pages it follows.
"""
import ctypes
import os

import numpy as np

from .build_oracle import build as _build

_lib = None

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(_build())
        lib.oracle_quantize_rows.argtypes = [_ptr, _i64, _i64, _ptr, _ptr]
        lib.oracle_quantize_tensor.argtypes = [_ptr, _i64, _i64, _ptr, _ptr]
        lib.oracle_trit5_row_bytes.argtypes = [_i64]
        lib.oracle_trit5_row_bytes.restype = _i64
        lib.oracle_trit5_row_stride.argtypes = [_i64]
        lib.oracle_trit5_row_stride.restype = _i64
        lib.oracle_int8_row_stride.argtypes = [_i64]
        lib.oracle_int8_row_stride.restype = _i64
        lib.oracle_pack_trit5.argtypes = [_ptr, _i64, _i64, _ptr, _ptr]
        lib.oracle_unpack_trit5.argtypes = [_ptr, _i64, _i64, _ptr]
        lib.oracle_unpack_trit5.restype = _i64
        lib.oracle_layout_int8.argtypes = [_ptr, _i64, _i64, _ptr]
        lib.oracle_matmul_int.argtypes = [_ptr, _ptr, _i64, _i64, _i64, _ptr, ctypes.c_int]
        lib.oracle_matmul_int.restype = ctypes.c_int
        lib.oracle_dequant.argtypes = [_ptr, _i64, _i64, _ptr, ctypes.c_float, _ptr]
        lib.oracle_lmhead.argtypes = [_ptr, _ptr, _i64, _i64, _ptr, _ptr, ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_sketch_signs.argtypes = [_ptr, _i64, _i64, _ptr, ctypes.c_int]
        lib.oracle_sketch_scale.argtypes = [_ptr, _i64, _i64, ctypes.c_int]
        lib.oracle_sketch_scale.restype = ctypes.c_double
        lib.oracle_sketch_plan.argtypes = [_ptr, _i64, ctypes.c_double, _ptr, _ptr, _ptr, _ptr, _ptr]
        lib.oracle_sketch_scores.argtypes = [_ptr, _ptr, _i64, _i64, ctypes.c_double, _ptr, _ptr, ctypes.c_int]
        lib.oracle_sketch_pick.argtypes = [_ptr, _ptr, _i64, _i64, _ptr, _ptr, _ptr, _ptr]
        lib.oracle_sketch_pick.restype = _i64
        lib.oracle_rmsnorm.argtypes = [_ptr, _ptr, _i64, _i64, ctypes.c_double, _ptr]
        lib.oracle_glu.argtypes = [_ptr, _ptr, _i64, _i64, ctypes.c_int, _ptr]
        lib.oracle_quantize_groups.argtypes = [_ptr, _i64, _i64, _i64, _ptr, _ptr]
        lib.oracle_gemv_grouped.argtypes = [_ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _ptr, _ptr, ctypes.c_int]
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def quantize_rows(x):
    """Per-row int8 quantisation of a 2-D fp32 array -> (int8 [m][k], fp32 [m])."""
    x, px = _c(np.atleast_2d(x), np.float32)
    m, k = x.shape
    q = np.empty((m, k), np.int8)
    s = np.empty(m, np.float32)
    _load().oracle_quantize_rows(px, m, k, q.ctypes.data, s.ctypes.data)
    return q, s


def quantize_tensor(w):
    """Per-tensor int8 quantisation of a 2-D fp32 array -> (int8 [n][k], fp32 scale)."""
    w, pw = _c(np.atleast_2d(w), np.float32)
    n, k = w.shape
    q = np.empty((n, k), np.int8)
    s = np.empty(1, np.float32)
    _load().oracle_quantize_tensor(pw, n, k, q.ctypes.data, s.ctypes.data)
    return q, np.float32(s[0])


def trit5_row_bytes(k: int) -> int:
    return int(_load().oracle_trit5_row_bytes(k))


def trit5_row_stride(k: int) -> int:
    return int(_load().oracle_trit5_row_stride(k))


def int8_row_stride(k: int) -> int:
    return int(_load().oracle_int8_row_stride(k))


def pack_trit5(t):
    """Trits [n][k] -> (packed bytes in the device layout, count of invalid trits)."""
    t, pt = _c(np.atleast_2d(t), np.int8)
    n, k = t.shape
    out = np.empty(n * trit5_row_stride(k), np.uint8)
    bad = np.zeros(1, np.int64)
    _load().oracle_pack_trit5(pt, n, k, out.ctypes.data, bad.ctypes.data)
    return out, int(bad[0])


def unpack_trit5(packed, n: int, k: int):
    """Packed device bytes -> (trits [n][k], count of bytes >= 243)."""
    p, pp = _c(packed, np.uint8)
    assert p.size == n * trit5_row_stride(k)
    t = np.empty((n, k), np.int8)
    invalid = _load().oracle_unpack_trit5(pp, n, k, t.ctypes.data)
    return t, int(invalid)


def layout_int8(q):
    """int8 codes [n][k] -> bytes in the device layout."""
    q, pq = _c(np.atleast_2d(q), np.int8)
    n, k = q.shape
    out = np.empty(n * int8_row_stride(k), np.int8)
    _load().oracle_layout_int8(pq, n, k, out.ctypes.data)
    return out


def matmul_int(x8, w, threads: int = 0):
    """Exact acc[m][n] = sum_k x8[m][k] * w[n][k] (int32; raises on overflow)."""
    x8, px = _c(np.atleast_2d(x8), np.int8)
    w, pw = _c(np.atleast_2d(w), np.int8)
    m, k = x8.shape
    n, k2 = w.shape
    assert k == k2
    acc = np.empty((m, n), np.int32)
    ovf = _load().oracle_matmul_int(px, pw, m, n, k, acc.ctypes.data, threads or max_threads())
    if ovf:
        raise OverflowError("integer dot product does not fit int32")
    return acc


def dequant(acc, sx, sw):
    """y[m][n] = fl32(acc * sx[m] * sw) formed in fp64."""
    acc, pa = _c(np.atleast_2d(acc), np.int32)
    sx, ps = _c(np.atleast_1d(sx), np.float32)
    m, n = acc.shape
    assert sx.size == m
    y = np.empty((m, n), np.float32)
    _load().oracle_dequant(pa, m, n, ps, ctypes.c_float(float(sw)), y.ctypes.data)
    return y


def lmhead(w_bf16, x, threads: int = 0):
    """Logits (fp64 [v]) and the first-max index of their fp32 roundings."""
    w, pw = _c(np.atleast_2d(w_bf16), np.uint16)
    x, px = _c(x, np.float32)
    v, k = w.shape
    assert x.size == k
    logits = np.empty(v, np.float64)
    idx = np.zeros(1, np.int32)
    _load().oracle_lmhead(pw, px, v, k, logits.ctypes.data, idx.ctypes.data, threads or max_threads())
    return logits, int(idx[0])


def sketch_signs(w_bf16, threads: int = 0):
    """Sign bits of a bf16 [v][k] table, word-major: uint32 [ceil(k/32)][v]."""
    w, pw = _c(np.atleast_2d(w_bf16), np.uint16)
    v, k = w.shape
    out = np.empty(((k + 31) // 32, v), np.uint32)
    _load().oracle_sketch_signs(pw, v, k, out.ctypes.data, threads or max_threads())
    return out


def sketch_scale(w_bf16, threads: int = 0):
    """c = mean |w| of the table (fp64)."""
    w, pw = _c(np.atleast_2d(w_bf16), np.uint16)
    v, k = w.shape
    return float(_load().oracle_sketch_scale(pw, v, k, threads or max_threads()))


def sketch_plan(x, c):
    """(top_idx [T], group_of [k] (-1 = exact), group_n [4], group_w [4] fp64)."""
    x, px = _c(x, np.float32)
    k = x.size
    top_idx = np.zeros(32, np.int32)
    ntop = np.zeros(1, np.int32)
    group_of = np.zeros(k, np.int32)
    group_n = np.zeros(4, np.int32)
    group_w = np.zeros(4, np.float64)
    _load().oracle_sketch_plan(px, k, ctypes.c_double(float(c)), top_idx.ctypes.data, ntop.ctypes.data,
                               group_of.ctypes.data, group_n.ctypes.data, group_w.ctypes.data)
    return top_idx[:int(ntop[0])], group_of, group_n, group_w


def sketch_scores(w_bf16, x, c, threads: int = 0):
    """Approximate scores (fp64 [v]) of steps 1 and 2 of the sketch head, and per word the sum of
    the magnitudes of the score's terms (fp64 [v])."""
    w, pw = _c(np.atleast_2d(w_bf16), np.uint16)
    x, px = _c(x, np.float32)
    v, k = w.shape
    assert x.size == k
    scores = np.empty(v, np.float64)
    mag = np.empty(v, np.float64)
    _load().oracle_sketch_scores(pw, px, v, k, ctypes.c_double(float(c)), scores.ctypes.data, mag.ctypes.data,
                                 threads or max_threads())
    return scores, mag


def sketch_pick(w_bf16, x, scores):
    """Step 3: (candidate mask [v] bool: the min(1024, v) best scores, exact logits fp64 [v]
    (0 off the candidates), pick)."""
    w, pw = _c(np.atleast_2d(w_bf16), np.uint16)
    x, px = _c(x, np.float32)
    scores, ps = _c(scores, np.float64)
    v, k = w.shape
    is_cand = np.zeros(v, np.uint8)
    logits = np.zeros(v, np.float64)
    idx = np.zeros(1, np.int32)
    _load().oracle_sketch_pick(pw, px, v, k, ps, is_cand.ctypes.data, logits.ctypes.data, idx.ctypes.data)
    return is_cand.astype(bool), logits, int(idx[0])


def sketch_head(w_bf16, x, threads: int = 0):
    """The whole sketch head: (pick, candidate mask, approximate scores, exact candidate logits)."""
    c = sketch_scale(w_bf16, threads)
    scores, _ = sketch_scores(w_bf16, x, c, threads)
    is_cand, logits, idx = sketch_pick(w_bf16, x, scores)
    return idx, is_cand, scores, logits


def rmsnorm(x, weight, eps=1e-5):
    """RMSNorm of every row in fp64: weight * x / sqrt(mean(x^2) + eps) -> fp64 [m][k]."""
    x, px = _c(np.atleast_2d(x), np.float32)
    w, pw = _c(weight, np.float32)
    m, k = x.shape
    assert w.size == k
    o = np.empty((m, k), np.float64)
    _load().oracle_rmsnorm(px, pw, m, k, ctypes.c_double(float(eps)), o.ctypes.data)
    return o


GLU_GELU_TANH = 1
GLU_SILU = 2


def glu(gate, up, act):
    """act(gate) * up in fp64 (act 1 = GeLU tanh form, 2 = SiLU)."""
    g, pg = _c(np.atleast_2d(gate), np.float32)
    u, pu = _c(np.atleast_2d(up), np.float32)
    assert g.shape == u.shape
    m, n = g.shape
    h = np.empty((m, n), np.float64)
    _load().oracle_glu(pg, pu, m, n, int(act), h.ctypes.data)
    return h


WEIGHT_GROUP = 128
ACT_GROUP = 32


def quantize_groups(x, group):
    """Group-wise int8 quantisation of the rows of a 2-D fp32 array:
    (int8 [m][k], fp32 [m][ceil(k/group)])."""
    x, px = _c(np.atleast_2d(x), np.float32)
    m, k = x.shape
    q = np.empty((m, k), np.int8)
    s = np.empty((m, (k + group - 1) // group), np.float32)
    _load().oracle_quantize_groups(px, m, k, int(group), q.ctypes.data, s.ctypes.data)
    return q, s


def gemv_grouped(w8, sw, x8, sx, threads: int = 0):
    """y (fp64 [m][n]) with weight scales per 128 and activation scales per 32
    columns, and sum_h |term| per output (the fp32 summation error scale)."""
    w8, pw = _c(w8, np.int8)
    x8, px = _c(np.atleast_2d(x8), np.int8)
    n, k = w8.shape
    m = x8.shape[0]
    assert x8.shape[1] == k
    sw, psw = _c(sw, np.float32)
    sx, psx = _c(np.atleast_2d(sx), np.float32)
    assert sw.shape == (n, (k + 127) // 128) and sx.shape == (m, (k + 31) // 32)
    y = np.empty((m, n), np.float64)
    b = np.empty((m, n), np.float64)
    _load().oracle_gemv_grouped(pw, psw, px, psx, m, n, k, y.ctypes.data, b.ctypes.data,
                                threads or max_threads())
    return y, b


__all__ = ["quantize_groups", "gemv_grouped", "WEIGHT_GROUP", "ACT_GROUP", "rmsnorm", "glu", "GLU_GELU_TANH", "GLU_SILU",
           "max_threads", "quantize_rows", "quantize_tensor", "trit5_row_bytes", "trit5_row_stride",
           "int8_row_stride", "pack_trit5", "unpack_trit5", "layout_int8", "matmul_int", "dequant",
           "lmhead", "sketch_signs", "sketch_scale", "sketch_plan", "sketch_scores", "sketch_pick", "sketch_head"]
