"""ctypes binding of libqmv (include/qmv.h) over PyTorch device tensors.

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch supplies device memory and the current stream.  If the library has
not been built, `load()` raises -- there is no fallback of any kind.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmv.so")

QMV_OK = 0
QMV_EINVAL = -1
QMV_ESHAPE = -2
QMV_EVALUE = -3
QMV_EHIP = -4
QMV_EUNSUPPORTED = -5
QMV_EWORKSPACE = -6

QMV_W_TERNARY5 = 1
QMV_W_INT8 = 2
QMV_W_INT8_G128 = 3
QMV_WEIGHT_GROUP = 128
QMV_ACT_GROUP = 32
QMV_MAX_GEMV_M = 16
QMV_PLAN_GEMV = 1
QMV_PLAN_PREFILL = 2
QMV_PLAN_GEMV_DOT = 3
QMV_PLAN_GEMV_SKIP_ZERO = 4

_c_i32, _c_i64, _c_u32, _c_ptr, _c_f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_float


class qmv_weight(ctypes.Structure):
    _fields_ = [("wtype", _c_i32), ("reserved", _c_i32), ("n", _c_i64), ("k", _c_i64),
                ("data", _c_ptr), ("scale", _c_ptr)]


class qmv_problem(ctypes.Structure):
    _fields_ = [("w", qmv_weight), ("x8", _c_ptr), ("sx", _c_ptr), ("m", _c_i64), ("y", _c_ptr),
                ("acc", _c_ptr)]


class qmv_ffn_layer(ctypes.Structure):
    _fields_ = [("gate", qmv_weight), ("up", qmv_weight), ("down", qmv_weight), ("norm", _c_ptr)]


class qmv_act(ctypes.Structure):
    _fields_ = [("x", _c_ptr), ("m", _c_i64), ("k", _c_i64), ("x8", _c_ptr), ("sx", _c_ptr)]


QMV_MAX_ACT_SETS = 8


class QmvError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, status_str(status), status))


_lib = None

# name -> (restype, argtypes); mirrors include/qmv.h
SIGNATURES = {
    "qmv_version": (ctypes.c_char_p, []),
    "qmv_status_str": (ctypes.c_char_p, [_c_i32]),
    "qmv_packed_bytes": (_c_i64, [_c_i32, _c_i64, _c_i64]),
    "qmv_pack_ternary": (_c_i32, [_c_ptr, _c_i64, _c_i64, _c_f32, _c_ptr, _c_ptr, _c_ptr,
                                  ctypes.POINTER(qmv_weight), _c_ptr]),
    "qmv_pack_int8": (_c_i32, [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, ctypes.POINTER(qmv_weight), _c_ptr]),
    "qmv_quantize_act": (_c_i32, [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr]),
    "qmv_quantize_act_many": (_c_i32, [ctypes.POINTER(qmv_act), _c_i32, _c_ptr]),
    "qmv_pack_int8_grouped": (_c_i32, [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, ctypes.POINTER(qmv_weight),
                                       _c_ptr]),
    "qmv_quantize_act_grouped": (_c_i32, [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr]),
    "qmv_workspace_bytes": (_c_i64, [ctypes.POINTER(qmv_problem), _c_i32]),
    "qmv_gemv_workspace_bytes": (_c_i64, [ctypes.POINTER(qmv_problem), _c_i32]),
    "qmv_prefill_workspace_bytes": (_c_i64, [ctypes.POINTER(qmv_problem), _c_i32]),
    "qmv_gemv": (_c_i32, [ctypes.POINTER(qmv_problem), _c_i32, _c_ptr, _c_i64, _c_ptr]),
    "qmv_gemm_prefill": (_c_i32, [ctypes.POINTER(qmv_problem), _c_i32, _c_ptr, _c_i64, _c_ptr]),
    "qmv_plan_create": (_c_i32, [_c_i32, ctypes.POINTER(qmv_problem), _c_i32, ctypes.POINTER(_c_ptr)]),
    "qmv_plan_workspace_bytes": (_c_i64, [_c_ptr]),
    "qmv_plan_upload": (_c_i32, [_c_ptr, _c_ptr, _c_i64, _c_ptr]),
    "qmv_plan_launch": (_c_i32, [_c_ptr, _c_ptr, _c_i64, _c_ptr]),
    "qmv_plan_destroy": (None, [_c_ptr]),
    "qmv_lmhead_workspace_bytes": (_c_i64, [_c_i64, _c_i64]),
    "qmv_lmhead_argmax": (_c_i32, [_c_ptr, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64,
                                   _c_ptr]),
    "qmv_lmhead_argmax_static": (_c_i32, [_c_ptr, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr]),
    "qmv_read_probe": (_c_i32, [_c_ptr, _c_i64, _c_ptr, _c_ptr]),
    "qmv_mfma_probe": (_c_i32, [_c_i32, _c_i32, _c_ptr, ctypes.POINTER(_c_i64), _c_ptr]),
    "qmv_rmsnorm_quantize": (_c_i32, [_c_ptr, _c_ptr, _c_i64, _c_i64, ctypes.c_float, _c_ptr, _c_ptr, _c_ptr]),
    "qmv_glu_quantize": (_c_i32, [_c_ptr, _c_ptr, _c_i64, _c_i64, _c_i32, _c_ptr, _c_ptr, _c_ptr]),
    "qmv_ffn_workspace_bytes": (_c_i64, [_c_i64, _c_i64]),
    "qmv_ffn_grid": (_c_i32, [ctypes.POINTER(_c_i32)]),
    "qmv_ffn_decode": (_c_i32, [ctypes.POINTER(qmv_ffn_layer), _c_i32, _c_ptr, ctypes.c_float, _c_i32, _c_ptr,
                                _c_i64, _c_ptr, _c_i64, _c_ptr, _c_ptr, _c_ptr]),
    "qmv_sketch_bytes": (_c_i64, [_c_i64, _c_i64]),
    "qmv_sketch_workspace_bytes": (_c_i64, [_c_i64, _c_i64]),
    "qmv_sketch_build": (_c_i32, [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_i64, _c_ptr]),
    "qmv_lmhead_sketch_argmax": (_c_i32, [_c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                          _c_ptr, _c_i64, _c_ptr]),
}


def load(path: str = LIB_PATH):
    """Load libqmv.so (built by ternary_matvec_amd.build); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError("libqmv.so not found at %s: build it with "
                               "`python -c 'import __graft_entry__; __graft_entry__.build()'`" % path)
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load().qmv_status_str(status).decode()


def version() -> str:
    return load().qmv_version().decode()


def _check(status, what):
    if status != QMV_OK:
        raise QmvError(status, what)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, dtype, what):
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError("%s must be a contiguous %s CUDA tensor" % (what, dtype))
    return t


def _alloc_aligned(nbytes, device, align=256):
    """A uint8 tensor of nbytes whose data pointer is `align`-aligned (plumbing only)."""
    raw = torch.empty(nbytes + align, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % align
    return raw[off:off + nbytes]


def qmv_packed_bytes(wtype: int, n: int, k: int) -> int:
    return int(load().qmv_packed_bytes(wtype, n, k))


class Weight:
    """A packed matrix: device bytes, device scale and its host descriptor."""

    def __init__(self, desc: qmv_weight, packed: torch.Tensor, scale: torch.Tensor):
        self.desc = desc
        self.packed = packed
        self.scale = scale

    @property
    def n(self):
        return int(self.desc.n)

    @property
    def k(self):
        return int(self.desc.k)

    @property
    def wtype(self):
        return int(self.desc.wtype)


def qmv_pack_ternary(trits, scale: float, packed=None, scale_out=None, bad_count=None, stream=None) -> Weight:
    _dev(trits, torch.int8, "trits")
    n, k = trits.shape
    nbytes = qmv_packed_bytes(QMV_W_TERNARY5, n, k)
    if packed is None:
        packed = _alloc_aligned(nbytes, trits.device, 16)
    if scale_out is None:
        scale_out = torch.empty(1, dtype=torch.float32, device=trits.device)
    desc = qmv_weight()
    _check(load().qmv_pack_ternary(_ptr(trits), n, k, float(scale), _ptr(packed), _ptr(scale_out),
                                   _ptr(bad_count), ctypes.byref(desc), _stream(stream)), "qmv_pack_ternary")
    return Weight(desc, packed, scale_out)


def qmv_pack_int8(w, packed=None, scale_out=None, stream=None) -> Weight:
    _dev(w, torch.float32, "w")
    n, k = w.shape
    nbytes = qmv_packed_bytes(QMV_W_INT8, n, k)
    if packed is None:
        packed = _alloc_aligned(nbytes, w.device, 16)
    if scale_out is None:
        scale_out = torch.empty(1, dtype=torch.float32, device=w.device)
    desc = qmv_weight()
    _check(load().qmv_pack_int8(_ptr(w), n, k, _ptr(packed), _ptr(scale_out), ctypes.byref(desc),
                                _stream(stream)), "qmv_pack_int8")
    return Weight(desc, packed, scale_out)


def qmv_quantize_act(x, x8=None, sx=None, stream=None):
    _dev(x, torch.float32, "x")
    m, k = x.shape
    if x8 is None:
        x8 = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if sx is None:
        sx = torch.empty(m, dtype=torch.float32, device=x.device)
    _check(load().qmv_quantize_act(_ptr(x), m, k, _ptr(x8), _ptr(sx), _stream(stream)), "qmv_quantize_act")
    return x8, sx


def qmv_pack_int8_grouped(w, packed=None, scales=None, stream=None) -> Weight:
    """fp32 [n][k] -> int8 codes in groups of 128 columns, one scale per group."""
    _dev(w, torch.float32, "w")
    n, k = w.shape
    nbytes = qmv_packed_bytes(QMV_W_INT8_G128, n, k)
    if packed is None:
        packed = _alloc_aligned(nbytes, w.device, 16)
    if scales is None:
        scales = torch.empty((n, (k + QMV_WEIGHT_GROUP - 1) // QMV_WEIGHT_GROUP), dtype=torch.float32,
                             device=w.device)
    desc = qmv_weight()
    _check(load().qmv_pack_int8_grouped(_ptr(w), n, k, _ptr(packed), _ptr(scales), ctypes.byref(desc),
                                        _stream(stream)), "qmv_pack_int8_grouped")
    return Weight(desc, packed, scales)


def qmv_quantize_act_grouped(x, x8=None, sx=None, stream=None):
    """fp32 [m][k] -> int8 codes with one scale per 32 columns: (x8 [m][k], sx [m][ceil(k/32)])."""
    _dev(x, torch.float32, "x")
    m, k = x.shape
    if x8 is None:
        x8 = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if sx is None:
        sx = torch.empty((m, (k + QMV_ACT_GROUP - 1) // QMV_ACT_GROUP), dtype=torch.float32, device=x.device)
    _check(load().qmv_quantize_act_grouped(_ptr(x), m, k, _ptr(x8), _ptr(sx), _stream(stream)),
           "qmv_quantize_act_grouped")
    return x8, sx


def act_array(sets):
    """[(x fp32 [m][k], x8 int8 [m][k], sx fp32 [m]), ...] -> a qmv_act array.  The array
    holds references to the tensors, so they live as long as it does."""
    arr = (qmv_act * len(sets))()
    arr._tensors = [tuple(s) for s in sets]
    for i, (x, x8, sx) in enumerate(sets):
        _dev(x, torch.float32, "x")
        _dev(x8, torch.int8, "x8")
        _dev(sx, torch.float32, "sx")
        m, k = x.shape
        if tuple(x8.shape) != (m, k) or sx.numel() != m:
            raise QmvError(QMV_ESHAPE, "act_array")
        arr[i] = qmv_act(x.data_ptr(), m, k, x8.data_ptr(), sx.data_ptr())
    return arr


def qmv_quantize_act_many(sets, stream=None):
    """qmv_quantize_act over several activation sets in one launch; `sets` is a
    list of (x, x8, sx) or an act_array."""
    arr = sets if isinstance(sets, ctypes.Array) else act_array(sets)
    _check(load().qmv_quantize_act_many(arr, len(arr), _stream(stream)), "qmv_quantize_act_many")
    return arr


class Problem:
    """y[m][n] = (x8 . W) * sx * scale for one weight matrix and m tokens."""

    def __init__(self, weight: Weight, x8, sx, y=None, acc=None):
        _dev(x8, torch.int8, "x8")
        _dev(sx, torch.float32, "sx")
        m = x8.shape[0]
        if y is None:
            y = torch.empty((m, weight.n), dtype=torch.float32, device=x8.device)
        self.weight, self.x8, self.sx, self.y, self.acc = weight, x8, sx, y, acc

    def struct(self) -> qmv_problem:
        p = qmv_problem()
        p.w = self.weight.desc
        p.x8 = self.x8.data_ptr()
        p.sx = self.sx.data_ptr()
        p.m = self.x8.shape[0]
        p.y = self.y.data_ptr()
        p.acc = None if self.acc is None else self.acc.data_ptr()
        return p


def problem_array(problems):
    """Problems -> a qmv_problem array.  The array holds references to the
    Problem objects (and so to their weights, activations and outputs): a plan
    launched after the caller dropped its Problems still writes into live
    tensors, never into memory the allocator has handed to someone else."""
    arr = (qmv_problem * len(problems))()
    for i, p in enumerate(problems):
        arr[i] = p.struct()
    arr._problems = list(problems)
    return arr


def qmv_gemv_workspace_bytes(arr) -> int:
    return int(load().qmv_gemv_workspace_bytes(arr, len(arr)))


def qmv_prefill_workspace_bytes(arr) -> int:
    return int(load().qmv_prefill_workspace_bytes(arr, len(arr)))


def qmv_workspace_bytes(arr) -> int:
    return int(load().qmv_workspace_bytes(arr, len(arr)))


def _as_array(problems):
    return problems if isinstance(problems, ctypes.Array) else problem_array(problems)


def _grouped(fn_name, ws_fn, problems, workspace, stream):
    arr = _as_array(problems)
    need = ws_fn(arr)
    if need < 0:
        raise QmvError(QMV_ESHAPE, fn_name)
    if workspace is None:
        dev = torch.device("cuda", torch.cuda.current_device())
        workspace = _alloc_aligned(max(need, 256), dev)
    _check(getattr(load(), fn_name)(arr, len(arr), _ptr(workspace), workspace.numel(), _stream(stream)), fn_name)
    return workspace


def qmv_gemv(problems, workspace=None, stream=None):
    """Grouped GEMV (1..16 tokens per problem): schedule, upload and launch in one call;
    returns the workspace used.  For a list launched again and again, use Plan."""
    return _grouped("qmv_gemv", qmv_gemv_workspace_bytes, problems, workspace, stream)


def qmv_gemm_prefill(problems, workspace=None, stream=None):
    """Grouped int8-MFMA GEMM for any number of tokens, in one call; returns the workspace used."""
    return _grouped("qmv_gemm_prefill", qmv_prefill_workspace_bytes, problems, workspace, stream)


class Plan:
    """qmv_plan_create/upload/launch/destroy: one problem list scheduled once, its
    tables uploaded into its workspace, then launched many times (kernels only)."""

    def __init__(self, kind, problems, workspace=None, stream=None):
        lib = load()
        self.arr = _as_array(problems)          # the host structs, and (through them) the tensors they name
        self._lib = lib
        self._h = _c_ptr()
        _check(lib.qmv_plan_create(kind, self.arr, len(self.arr), ctypes.byref(self._h)), "qmv_plan_create")
        self.kind = kind
        need = int(lib.qmv_plan_workspace_bytes(self._h))
        if workspace is None:
            dev = torch.device("cuda", torch.cuda.current_device())
            workspace = _alloc_aligned(max(need, 256), dev)
        self.workspace = workspace
        self.upload(stream)

    def upload(self, stream=None):
        _check(self._lib.qmv_plan_upload(self._h, _ptr(self.workspace), self.workspace.numel(), _stream(stream)),
               "qmv_plan_upload")

    def launch(self, stream=None):
        _check(self._lib.qmv_plan_launch(self._h, _ptr(self.workspace), self.workspace.numel(), _stream(stream)),
               "qmv_plan_launch")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.qmv_plan_destroy(h)
            self._h = None


def gemv_plan(problems, workspace=None, stream=None, dot_only=False, skip_zero=False):
    kind = QMV_PLAN_GEMV_SKIP_ZERO if skip_zero else QMV_PLAN_GEMV_DOT if dot_only else QMV_PLAN_GEMV
    return Plan(kind, problems, workspace, stream)


def prefill_plan(problems, workspace=None, stream=None):
    return Plan(QMV_PLAN_PREFILL, problems, workspace, stream)


def qmv_lmhead_workspace_bytes(v: int, k: int) -> int:
    return int(load().qmv_lmhead_workspace_bytes(v, k))


def qmv_read_probe(buf, out, stream=None):
    """Measurement aid: read a device tensor once (16-byte loads) and fold it into out[0]
    only on a fixed key; timed beside qmv_gemv it gives the achievable HBM read rate."""
    import torch
    assert buf.is_cuda and out.is_cuda and out.dtype in (torch.int32, torch.uint32) and out.numel() >= 1
    _check(load().qmv_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), out.data_ptr(),
                                 _stream(stream)), "qmv_read_probe")


def qmv_mfma_probe(kind, iters, out, stream=None) -> int:
    """Launch the matrix-instruction yardstick; returns the launch's int8 operations."""
    ops = _c_i64(0)
    _check(load().qmv_mfma_probe(int(kind), int(iters), _ptr(out), ctypes.byref(ops), _stream(stream)),
           "qmv_mfma_probe")
    return int(ops.value)


def qmv_lmhead_argmax(w_bf16, x, logits=None, idx=None, max_logit=None, workspace=None, want_logits=False,
                      stream=None):
    """Returns (idx tensor [1] int32, max_logit tensor [1] fp32, logits or None)."""
    if w_bf16.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("w_bf16 must hold bf16 bit patterns")
    _dev(x, torch.float32, "x")
    v, k = w_bf16.shape
    dev = x.device
    if idx is None:
        idx = torch.empty(1, dtype=torch.int32, device=dev)
    if max_logit is None:
        max_logit = torch.empty(1, dtype=torch.float32, device=dev)
    if logits is None and want_logits:
        logits = torch.empty(v, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _alloc_aligned(max(qmv_lmhead_workspace_bytes(v, k), 256), dev)
    _check(load().qmv_lmhead_argmax(_ptr(w_bf16), _ptr(x), v, k, _ptr(idx), _ptr(max_logit), _ptr(logits),
                                    _ptr(workspace), workspace.numel(), _stream(stream)), "qmv_lmhead_argmax")
    return idx, max_logit, logits


def qmv_lmhead_argmax_static(w_bf16, x, logits=None, idx=None, max_logit=None, want_logits=False, stream=None):
    """qmv_lmhead_argmax with the library's static scratch instead of a workspace:
    returns (idx tensor [1] int32, max_logit tensor [1] fp32, logits or None)."""
    if w_bf16.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("w_bf16 must hold bf16 bit patterns")
    _dev(x, torch.float32, "x")
    v, k = w_bf16.shape
    dev = x.device
    if idx is None:
        idx = torch.empty(1, dtype=torch.int32, device=dev)
    if max_logit is None:
        max_logit = torch.empty(1, dtype=torch.float32, device=dev)
    if logits is None and want_logits:
        logits = torch.empty(v, dtype=torch.float32, device=dev)
    _check(load().qmv_lmhead_argmax_static(_ptr(w_bf16), _ptr(x), v, k, _ptr(idx), _ptr(max_logit), _ptr(logits),
                                           _stream(stream)), "qmv_lmhead_argmax_static")
    return idx, max_logit, logits


def qmv_sketch_bytes(v: int, k: int) -> int:
    return int(load().qmv_sketch_bytes(v, k))


def qmv_sketch_workspace_bytes(v: int, k: int) -> int:
    return int(load().qmv_sketch_workspace_bytes(v, k))


def qmv_sketch_build(w_bf16, sketch=None, stream=None):
    """Builds the sketch tables of a [v][k] bf16 table; returns the uint8 sketch buffer."""
    if w_bf16.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("w_bf16 must hold bf16 bit patterns")
    v, k = w_bf16.shape
    nbytes = qmv_sketch_bytes(v, k)
    if nbytes < 0:
        raise QmvError(-2, "qmv_sketch_bytes")
    if sketch is None:
        sketch = _alloc_aligned(nbytes, w_bf16.device)
    _check(load().qmv_sketch_build(_ptr(w_bf16), v, k, _ptr(sketch), sketch.numel(), _stream(stream)),
           "qmv_sketch_build")
    return sketch


def sketch_workspace(v: int, k: int, device):
    """A zero-filled, 256-byte aligned sketch workspace (the state it carries
    between tokens starts at zero; every call leaves it ready for the next)."""
    nbytes = qmv_sketch_workspace_bytes(v, k)
    if nbytes < 0:
        raise QmvError(-2, "qmv_sketch_workspace_bytes")
    ws = _alloc_aligned(nbytes, device)
    ws.zero_()
    return ws


def qmv_lmhead_sketch_argmax(w_bf16, sketch, x, idx=None, max_logit=None, candidates=None, scores=None,
                             workspace=None, want_scores=False, stream=None):
    """Returns (idx [1] int32, max_logit [1] fp32, candidates [1] int32, scores [v] fp32 or None)."""
    if w_bf16.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("w_bf16 must hold bf16 bit patterns")
    _dev(x, torch.float32, "x")
    v, k = w_bf16.shape
    dev = x.device
    if idx is None:
        idx = torch.empty(1, dtype=torch.int32, device=dev)
    if max_logit is None:
        max_logit = torch.empty(1, dtype=torch.float32, device=dev)
    if candidates is None:
        candidates = torch.empty(1, dtype=torch.int32, device=dev)
    if scores is None and want_scores:
        scores = torch.empty(v, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = sketch_workspace(v, k, dev)
    _check(load().qmv_lmhead_sketch_argmax(_ptr(w_bf16), _ptr(sketch), _ptr(x), v, k, _ptr(idx), _ptr(max_logit),
                                           _ptr(candidates), _ptr(scores), _ptr(workspace), workspace.numel(),
                                           _stream(stream)), "qmv_lmhead_sketch_argmax")
    return idx, max_logit, candidates, scores


QMV_ACT_GELU_TANH = 1
QMV_ACT_SILU = 2


def qmv_rmsnorm_quantize(x, weight, eps=1e-5, x8=None, sx=None, stream=None):
    """RMSNorm then per-row int8 of a [m][k] fp32 tensor; returns (x8, sx)."""
    _dev(x, torch.float32, "x")
    _dev(weight, torch.float32, "weight")
    x2 = x if x.dim() == 2 else x.view(1, -1)
    m, k = x2.shape
    if weight.numel() != k:
        raise QmvError(-2, "qmv_rmsnorm_quantize")
    if x8 is None:
        x8 = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if sx is None:
        sx = torch.empty(m, dtype=torch.float32, device=x.device)
    _check(load().qmv_rmsnorm_quantize(_ptr(x2), _ptr(weight), m, k, ctypes.c_float(eps), _ptr(x8), _ptr(sx),
                                       _stream(stream)), "qmv_rmsnorm_quantize")
    return x8, sx


def qmv_glu_quantize(gate, up, act=QMV_ACT_GELU_TANH, x8=None, sx=None, stream=None):
    """act(gate) * up then per-row int8 of [m][n] fp32 tensors; returns (x8, sx)."""
    _dev(gate, torch.float32, "gate")
    _dev(up, torch.float32, "up")
    g2 = gate if gate.dim() == 2 else gate.view(1, -1)
    u2 = up if up.dim() == 2 else up.view(1, -1)
    if g2.shape != u2.shape:
        raise QmvError(-2, "qmv_glu_quantize")
    m, n = g2.shape
    if x8 is None:
        x8 = torch.empty((m, n), dtype=torch.int8, device=gate.device)
    if sx is None:
        sx = torch.empty(m, dtype=torch.float32, device=gate.device)
    _check(load().qmv_glu_quantize(_ptr(g2), _ptr(u2), m, n, int(act), _ptr(x8), _ptr(sx), _stream(stream)),
           "qmv_glu_quantize")
    return x8, sx


QMV_FFN_OK = 0
QMV_FFN_CANCELLED = 1
QMV_FFN_TIMEOUT = 2
QMV_FFN_LAUNCH_LAYERS = 32
QMV_FFN_TRACE_STAMPS = 12
QMV_FFN_MAX_HIDDEN = 8192
QMV_FFN_MAX_INTER = 65536


def qmv_ffn_workspace_bytes(hidden: int, inter: int) -> int:
    return int(load().qmv_ffn_workspace_bytes(hidden, inter))


def qmv_ffn_grid() -> int:
    g = _c_i32(0)
    _check(load().qmv_ffn_grid(ctypes.byref(g)), "qmv_ffn_grid")
    return int(g.value)


def ffn_layer_array(layers):
    """layers: sequence of (gate Weight, up Weight, down Weight, norm tensor).  The
    array holds references to them, so they live as long as it does."""
    arr = (qmv_ffn_layer * len(layers))()
    arr._layers = [tuple(l) for l in layers]
    for i, (g, u, d, norm) in enumerate(layers):
        _dev(norm, torch.float32, "norm")
        arr[i].gate, arr[i].up, arr[i].down = g.desc, u.desc, d.desc
        arr[i].norm = norm.data_ptr()
    return arr


def ffn_workspace(hidden: int, inter: int, device):
    """A zero-filled, 256-byte aligned workspace for qmv_ffn_decode."""
    n = qmv_ffn_workspace_bytes(hidden, inter)
    if n < 0:
        raise QmvError(QMV_ESHAPE, "qmv_ffn_workspace_bytes")
    ws = _alloc_aligned(n, device)
    ws.zero_()
    return ws


def qmv_ffn_decode(layers, h, eps=1e-6, act=QMV_ACT_GELU_TANH, workspace=None, status=None, cancel=None,
                   spin_limit=0, trace=None, stream=None):
    """The feed-forward half of len(layers) layers for one token, h updated in
    place.  layers: a ctypes qmv_ffn_layer array (ffn_layer_array).  Returns the
    status tensor (1 int32, device; read it after synchronising)."""
    _dev(h, torch.float32, "h")
    if not isinstance(layers, ctypes.Array):
        layers = ffn_layer_array(layers)
    if workspace is None:
        workspace = ffn_workspace(int(layers[0].gate.k), int(layers[0].gate.n), h.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=h.device)
    _check(load().qmv_ffn_decode(layers, len(layers), _ptr(h), ctypes.c_float(eps), int(act), _ptr(workspace),
                                 workspace.numel(), None if cancel is None else ctypes.c_void_p(cancel.data_ptr()),
                                 int(spin_limit), _ptr(status), _ptr(trace), _stream(stream)), "qmv_ffn_decode")
    return status
