"""Benchmark of the quantized matvec hot path on one MI355X.

Headline workload: batch-1 ternary decode over Gemma-3-1B-shaped weights,
26 layers x {q, k, v, gate, up, down} = 156 matrices, trits iid with
P(-1, 0, +1) = (0.3, 0.4, 0.3), one scale per matrix, x ~ N(0, 1).  One step:
  qmv_quantize_act_many on the 130 activation rows of K = 1152 and the 26 rows
  of K = 6912 (one launch), then one grouped qmv_gemv (a plan) over the 156
  problems.
Weights rotate over 8 full copies so the 256 MB Infinity Cache cannot hold the
working set.  `value` = algorithmic bytes per step / step time.

Timing: every GPU figure is the median of 5 repetitions, each timing R
back-to-back calls (R >= 100 for launches under a millisecond) between two HIP
events recorded on the stream the kernels run on.  The grouped GEMV's launch
time (roofline.achieved) is timed the same way on its own, so it is never
longer than the step it belongs to; its rocprofv3 kernel-trace median agrees
with it (the profiles' command is `--profile-set`, which runs only the launches
the profiles describe).

Also reported by default: the "+o_proj" decode step (182 matrices), the
BitNet-b1.58-large-shaped decode (168 matrices) at 1, 4 and 16 tokens with the
kernel that served each and the dot-product plan beside it, the 512-token
prefill through one prefill plan launch (int8 TOPS against the published int8
matrix-core peak and against a register-only matrix-instruction ceiling
measured in the same run), and the CPU oracle timed on the host's cores on bounded
samples of each configuration.

Opt-in (--extras NAME,... or all; never part of the default run): the weight-copy
sweep, chained per-matrix launches, the quantiser alone, host overhead per
launch, the feed-forward half as a launch-per-step chain and as one persistent
launch, zero-group skipping, the 262144 x 1152 bf16 output layer with greedy
argmax, the sketch head, the 768 x 288 int8 GEMV, the group-scaled int8 decode
and the BitNet decode at 1..16 tokens.
Each extra prints its name before it starts.
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, datasheet
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA, datasheet
GEMV_SOURCES = ("k_gemv_stream.hip", "unpack.hpp", "zform.hpp", "qmv_internal.hpp")
GEMV_COUNTERS = os.path.join(ROOT, "profiles", "k_gemv_stream_counters.json")
N_REP = 5
WARM_MS = 200.0   # GPU time of back-to-back calls before a timed row's repetitions
EXTRAS = ("decode_copies_sweep", "decode_chained", "quantize_step", "host_overhead", "ffn", "zero_skip", "lmhead",
          "lmhead_sketch", "int8_gemv", "groupscale_decode", "bitnet_decode_all")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="back-to-back steps per repetition (at least 100)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="GPU time of back-to-back calls before each timed row's repetitions (0: none; counter "
                         "runs, whose figures do not depend on it, use 0)")
    ap.add_argument("--copies", type=int, default=8, help="weight copies rotated to defeat the MALL")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extras", default="",
                    help="comma-separated extra measurements to run after the headline and prefill (or 'all'): "
                         + ", ".join(EXTRAS))
    ap.add_argument("--profile-set", action="store_true",
                    help="only the launches the kernel profiles describe, each kernel name from one workload: "
                         "decode steps, BitNet decode at 4 and 16 tokens, prefill passes, and the extras named "
                         "with --extras in their profiled form (the persistent feed-forward launch alone, the "
                         "zero-skip plan alone); no CPU baselines of the other configurations")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU-oracle time for the headline")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB five times: the "
                         "known-size kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    args.extras = list(EXTRAS) if args.extras == "all" else [e for e in args.extras.split(",") if e]
    for e in args.extras:
        if e not in EXTRAS:
            ap.error("unknown extra %r (known: %s)" % (e, ", ".join(EXTRAS)))
    return args


def median_time(fn, reps, stream, warm=3, n_rep=N_REP, warm_ms=None):
    """Median (over n_rep repetitions) of the time per call of `reps`
    back-to-back calls fn(i), in ms, with every repetition's value.  Before
    the repetitions: `warm` calls, then blocks of `reps` calls until warm_ms of
    GPU time has passed (back-to-back times keep falling for tens of ms after a
    pause: clocks and caches settle), so the repetitions see steady state."""
    import torch
    for i in range(warm):
        fn(i)
    warm_ms = WARM_MS if warm_ms is None else warm_ms
    spent = 0.0
    while spent < warm_ms:
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(reps):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        spent += t0.elapsed_time(t1)
    vals = []
    for r in range(n_rep):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(reps):
            fn(r * reps + i)
        t1.record(stream)
        torch.cuda.synchronize()
        vals.append(t0.elapsed_time(t1) / reps)
    return float(np.median(vals)), vals


def us(ms):
    return round(ms * 1e3, 3)


# ---------------------------------------------------------------------------
# Workload construction
# ---------------------------------------------------------------------------

class DecodeStack:
    """A stack of ternary matrices packed on the GPU (rotating copies), with
    its activations and one plan per copy.  zero_groups: the activations get
    80% zero groups of 4 columns (the ternary page's "What is next")."""

    def __init__(self, mats, layers, config_id, m, copies, dev, zero_groups=False):
        import torch
        from ternary_matvec_amd import qmv, synth
        self.mats, self.layers, self.m, self.copies = mats, layers, m, copies
        self.config_id = config_id
        self.specs = []
        ks = sorted(set(k for _, _, k in mats))
        self.x = {}                # K -> fp32 [rows*m][K] on device (host copy kept for the oracle)
        self.x_host = {}
        rows_per_k = {k: 0 for k in ks}
        for layer in range(layers):
            for mid, (name, n, k) in enumerate(mats):
                self.specs.append((layer, mid, name, n, k, rows_per_k[k]))
                rows_per_k[k] += 1
        for k in ks:
            xs = []
            for (layer, mid, _, _, kk, _) in self.specs:
                if kk != k:
                    continue
                x = synth.normal(synth.stream_seed(config_id, layer, mid, synth.TAG_ACT), (m, kk))
                if zero_groups:
                    x[synth.zero_groups(synth.stream_seed(config_id, layer, mid, synth.TAG_MISC), (m, kk))] = 0.0
                xs.append(x)
            self.x_host[k] = np.concatenate(xs, axis=0)
            self.x[k] = torch.from_numpy(self.x_host[k]).to(dev)
        self.x8, self.sx = {}, {}
        for k in ks:
            self.x8[k] = torch.empty(self.x[k].shape, dtype=torch.int8, device=dev)
            self.sx[k] = torch.empty(self.x[k].shape[0], dtype=torch.float32, device=dev)
        # every width's activations quantised by one launch
        self.acts = qmv.act_array([(self.x[k], self.x8[k], self.sx[k]) for k in ks])
        qmv.qmv_quantize_act_many(self.acts)
        total_packed = sum(qmv.qmv_packed_bytes(qmv.QMV_W_TERNARY5, n, k) for (_, _, _, n, k, _) in self.specs)
        self.packed_bytes = total_packed
        self.pool = [qmv._alloc_aligned(total_packed, dev, 256) for _ in range(copies)]
        self.scales = torch.empty(len(self.specs), dtype=torch.float32, device=dev)
        self.y = {}
        off = 0
        descs = []
        for i, (layer, mid, name, n, k, slot) in enumerate(self.specs):
            nb = qmv.qmv_packed_bytes(qmv.QMV_W_TERNARY5, n, k)
            t = synth.trits_torch(synth.stream_seed(config_id, layer, mid, synth.TAG_WEIGHT), (n, k), device=dev)
            s = synth.ternary_scale(synth.stream_seed(config_id, layer, mid, synth.TAG_SCALE))
            w = qmv.qmv_pack_ternary(t, s, packed=self.pool[0][off:off + nb], scale_out=self.scales[i:i + 1])
            descs.append((off, nb, w))
            self.y[i] = torch.empty((m, n), dtype=torch.float32, device=dev)
            off += nb
            del t
        torch.cuda.synchronize()
        for c in range(1, copies):
            self.pool[c].copy_(self.pool[0])
        torch.cuda.synchronize()
        self.arrays, self.plans = [], []
        for c in range(copies):
            probs = []
            for i, (off_i, nb, w) in enumerate(descs):
                layer, mid, name, n, k, slot = self.specs[i]
                wc = qmv.Weight(qmv.qmv_weight(w.desc.wtype, 0, n, k, self.pool[c][off_i:].data_ptr(),
                                               self.scales[i:i + 1].data_ptr()),
                                self.pool[c][off_i:off_i + nb], self.scales[i:i + 1])
                probs.append(qmv.Problem(wc, self.x8[k][slot * m:(slot + 1) * m], self.sx[k][slot * m:(slot + 1) * m],
                                         y=self.y[i]))
            arr = qmv.problem_array(probs)
            self.arrays.append(arr)
            self.plans.append(qmv.gemv_plan(arr) if m <= qmv.QMV_MAX_GEMV_M else None)
        torch.cuda.synchronize()

    def weight_bytes(self):
        return sum(n * ((k + 4) // 5) for (_, _, _, n, k, _) in self.specs)

    def weights(self):
        return sum(n * k for (_, _, _, n, k, _) in self.specs)

    def gemv_bytes(self):
        """Bytes one grouped GEMV must move: packed weights at 5 trits/byte,
        int8 activations in, fp32 outputs out, one scale per matrix and token."""
        m = self.m
        return sum(n * ((k + 4) // 5) + m * k + 4 * m * n + 4 + 4 * m for (_, _, _, n, k, _) in self.specs)

    def quant_bytes(self):
        return sum(5 * v.numel() + 4 * v.shape[0] for v in self.x.values())

    def step_bytes(self):
        return self.gemv_bytes() + self.quant_bytes()

    def macs(self):
        return sum(self.m * n * k for (_, _, _, n, k, _) in self.specs)

    def plan_kind(self, kind, copies=None):
        """Plans of another kind (dot-product kernels, zero-skip) over the same problems."""
        from ternary_matvec_amd import qmv
        copies = copies or self.copies
        return [qmv.Plan(kind, self.arrays[c]) for c in range(copies)]


def route_of(m):
    """The kernel a qmv_gemv plan runs for ternary problems of m tokens whose
    staged activations fit the matrix-core kernel's LDS (the library's routing)."""
    if m == 1:
        return "k_gemv_stream<1,1> (v_dot2 on staged Z operands)"
    if m <= 16:
        mt = 2 if m <= 2 else 4 if m <= 4 else 8 if m <= 8 else 16
        return "k_gemv_mx<%d> (v_mfma_i32_16x16x64_i8 on prefix-quotient bytes)" % mt
    return "k_gemv (workgroup tiles, v_dot4 on reordered planes)"


# ---------------------------------------------------------------------------
# Headline: decode steps
# ---------------------------------------------------------------------------

def time_decode(stack, reps, warm, stream, plans=None):
    """(step ms, GEMV-only ms): whole steps (quantise + grouped GEMV), and the
    grouped GEMV alone, both median of 5 x reps back-to-back."""
    from ternary_matvec_amd import qmv
    plans = plans or stack.plans
    nc = len(plans)

    def step(i):
        qmv.qmv_quantize_act_many(stack.acts, stream=stream)
        plans[i % nc].launch(stream)

    def gemv(i):
        plans[i % nc].launch(stream)

    step_ms, step_all = median_time(step, reps, stream, warm)
    gemv_ms, gemv_all = median_time(gemv, reps, stream, warm)
    return step_ms, gemv_ms, step_all, gemv_all


def time_read_ceiling(stack, reps, stream):
    """The plain-read yardstick (qmv_read_probe) over the same weight copies,
    rotated like the GEMV's: the HBM read rate this machine reaches on them."""
    import torch
    from ternary_matvec_amd import qmv
    out = torch.zeros(1, dtype=torch.int32, device=stack.pool[0].device)
    ms, _ = median_time(lambda i: qmv.qmv_read_probe(stack.pool[i % stack.copies], out, stream=stream), reps, stream)
    return stack.pool[0].numel() / ms / 1e6, ms


def gemv_source_hash():
    """sha256 over the sources of the streaming GEMV kernel (counter records name the hash they
    were taken with)."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, "ternary_matvec_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def gemv_traffic():
    """HBM bytes per launch of the streaming GEMV from the committed rocprofv3 counter record:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over the headline launch's dispatches),
    each scaled by the factor the same counter gave for a plain copy of known size.  None when the
    record is missing or was taken with different kernel sources."""
    try:
        with open(GEMV_COUNTERS) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != gemv_source_hash():
        return None
    kib = rec["fetch_kib"] * rec["fetch_factor"] + rec["write_kib"] * rec["write_factor"]
    return int(round(kib * 1024))


# ---------------------------------------------------------------------------
# Prefill
# ---------------------------------------------------------------------------

class PrefillStack:
    """The decode stack's weights (copy 0) with 512-token activations per matrix."""

    def __init__(self, stack, m, dev):
        import torch
        from ternary_matvec_amd import qmv, synth
        self.stack, self.m = stack, m
        ks = sorted(stack.x.keys())
        self.x, self.x8, self.sx = {}, {}, {}
        for k in ks:
            rows = [s for s in stack.specs if s[4] == k]
            xk = torch.empty((len(rows) * m, k), dtype=torch.float32, device=dev)
            for (layer, mid, name, n, kk, slot) in rows:
                xk[slot * m:(slot + 1) * m] = synth.normal_torch(
                    synth.stream_seed(synth.CONFIG_GEMMA_PREFILL, layer, mid, synth.TAG_ACT), (m, k), device=dev)
            self.x[k] = xk
            self.x8[k] = torch.empty(xk.shape, dtype=torch.int8, device=dev)
            self.sx[k] = torch.empty(xk.shape[0], dtype=torch.float32, device=dev)
        self.acts = qmv.act_array([(self.x[k], self.x8[k], self.sx[k]) for k in ks])
        self.y = {}
        probs = []
        pool = stack.pool[0]
        off = 0
        for i, (layer, mid, name, n, k, slot) in enumerate(stack.specs):
            nb = qmv.qmv_packed_bytes(qmv.QMV_W_TERNARY5, n, k)
            w = qmv.Weight(qmv.qmv_weight(qmv.QMV_W_TERNARY5, 0, n, k, pool[off:].data_ptr(),
                                          stack.scales[i:i + 1].data_ptr()), pool[off:off + nb], stack.scales[i:i + 1])
            off += nb
            self.y[i] = torch.empty((m, n), dtype=torch.float32, device=dev)
            probs.append(qmv.Problem(w, self.x8[k][slot * m:(slot + 1) * m], self.sx[k][slot * m:(slot + 1) * m],
                                     y=self.y[i]))
        self.arr = qmv.problem_array(probs)
        self.plan = qmv.prefill_plan(self.arr)
        qmv.qmv_quantize_act_many(self.acts)
        torch.cuda.synchronize()

    def ops(self):
        return 2 * sum(self.m * n * k for (_, _, _, n, k, _) in self.stack.specs)

    def bytes(self):
        """Algorithmic bytes of one pass: packed weights, int8 activations in, fp32 outputs out."""
        m = self.m
        return sum(n * ((k + 4) // 5) + m * k + 4 * m * n + 4 + 4 * m for (_, _, _, n, k, _) in self.stack.specs)

    def quant_bytes(self):
        return sum(5 * v.numel() + 4 * v.shape[0] for v in self.x.values())


def mfma_ceiling(dev, stream):
    """The int8 matrix-instruction rate of this GPU with no memory traffic
    (qmv_mfma_probe), for both instruction shapes; TOPS."""
    import torch
    from ternary_matvec_amd import qmv
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {}
    for kind, name in ((0, "v_mfma_i32_16x16x64_i8"), (1, "v_mfma_i32_32x32x32_i8")):
        iters = 2048 if kind == 0 else 1024
        ops = qmv.qmv_mfma_probe(kind, iters, out, stream=stream)
        ms, _ = median_time(lambda i: qmv.qmv_mfma_probe(kind, iters, out, stream=stream), 10, stream)
        res[name] = round(ops / ms / 1e9, 1)
    return res


def bench_prefill(stack, dev, stream, reps=20):
    import torch
    from ternary_matvec_amd import qmv
    ps = PrefillStack(stack, 512, dev)
    kern_ms, kern_all = median_time(lambda i: ps.plan.launch(stream), reps, stream)
    quant_ms, _ = median_time(lambda i: qmv.qmv_quantize_act_many(ps.acts, stream=stream), reps, stream)
    ceil = mfma_ceiling(dev, stream)
    tops = ps.ops() / kern_ms / 1e9
    out = {"workload": "ternary prefill, 512 tokens x Gemma-3-1B shapes x26 layers (156 matrices)",
           "kernel": "k_prefill (v_mfma_i32_32x32x32_i8)", "prefill_us": us(kern_ms),
           "prefill_us_reps": [us(v) for v in kern_all],
           "quantize_us": us(quant_ms), "quantize_GB/s": round(ps.quant_bytes() / quant_ms / 1e6, 1),
           "TOPS": round(tops, 1), "frac_int8_mfma_peak": round(tops / INT8_PEAK_TOPS, 4),
           "measured_mfma_ceiling_TOPS": ceil,
           "frac_of_measured_ceiling": round(tops / ceil["v_mfma_i32_32x32x32_i8"], 4),
           "GB/s": round(ps.bytes() / kern_ms / 1e6, 1), "ops_per_pass": ps.ops(), "bytes_per_pass": ps.bytes()}
    del ps
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# Extras
# ---------------------------------------------------------------------------

def copies_sweep(stack, reps, stream):
    """GEMV GB/s with the weights rotated over C = 1, 2, 4, 8 copies: the rate must be
    flat once the rotating set (C x 137.5 MB) is well past the 256 MB Infinity Cache."""
    out = {}
    for c_count in (1, 2, 4, 8):
        if c_count > stack.copies:
            break
        ms, _ = median_time(lambda i: stack.plans[i % c_count].launch(stream), reps, stream)
        out["C%d" % c_count] = {"gemv_us": us(ms), "GB/s": round(stack.gemv_bytes() / ms / 1e6, 1)}
    return out


def chained(stack, reps, stream, copies=4):
    """The step as stream-ordered launches instead of one grouped launch: 156 (one per
    matrix) or 78 (q/k/v and gate/up grouped per layer, down alone)."""
    import torch
    from ternary_matvec_amd import qmv
    copies = min(copies, stack.copies)
    per_layer = len(stack.mats)
    groups = {"156": [], "78": []}
    for c in range(copies):
        arr = stack.arrays[c]
        base = ctypes.addressof(arr)
        size = ctypes.sizeof(qmv.qmv_problem)
        one, grouped = [], []
        for i in range(len(arr)):
            sub = (qmv.qmv_problem * 1).from_address(base + i * size)
            one.append(qmv.gemv_plan(sub, stream=stream))
        for lay in range(len(arr) // per_layer):
            for lo, hi in ((0, 3), (3, 5), (5, 6)):
                sub = (qmv.qmv_problem * (hi - lo)).from_address(base + (lay * per_layer + lo) * size)
                grouped.append(qmv.gemv_plan(sub, stream=stream))
        groups["156"].append(one)
        groups["78"].append(grouped)
    torch.cuda.synchronize()
    out = {}
    for name, per_copy in groups.items():
        def step(i):
            for plan in per_copy[i % copies]:
                plan.launch(stream)
        ms, _ = median_time(step, reps, stream)
        # the same launches replayed from a graph per weight copy: the GPU's own cost
        # of the dependent chain, without the host's per-call time
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cap = torch.cuda.current_stream()
                for plan in per_copy[c]:
                    plan.launch(cap)
            graphs.append(g)
        torch.cuda.synchronize()
        gms, _ = median_time(lambda i: graphs[i % copies].replay(), reps, stream)
        out["launches_%s" % name] = {"step_us": us(ms), "GB/s": round(stack.gemv_bytes() / ms / 1e6, 1),
                                     "graph_step_us": us(gms),
                                     "graph_GB/s": round(stack.gemv_bytes() / gms / 1e6, 1)}
        del graphs
        torch.cuda.synchronize()
    return out


def host_overhead(stack, stream, calls=200):
    """Host time per call, measured on the host with the GPU kept busy: a plan
    launch (Python -> ctypes -> qmv_plan_launch -> hipLaunchKernel), and the
    one-shot qmv_gemv that schedules, uploads and launches per call."""
    import torch
    from ternary_matvec_amd import qmv
    plan = stack.plans[0]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        plan.launch(stream)
    t_plan = (time.perf_counter() - t0) / calls
    torch.cuda.synchronize()
    n1 = 20
    wss = [qmv._alloc_aligned(qmv.qmv_gemv_workspace_bytes(stack.arrays[0]), stack.pool[0].device)
           for _ in range(n1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n1):
        qmv.qmv_gemv(stack.arrays[0], workspace=wss[i], stream=stream)
    t_one = (time.perf_counter() - t0) / n1
    torch.cuda.synchronize()
    return {"plan_launch_host_us": round(t_plan * 1e6, 2), "one_shot_qmv_gemv_host_us": round(t_one * 1e6, 1),
            "note": "host time per call of a 156-problem list (the one-shot call schedules the 156 problems "
                    "and uploads the table each time)"}


def bench_o_proj(dev, stream, reps, copies):
    """The decode step with each layer's o projection (1152 x 1024) added: 182 matrices."""
    import torch
    from ternary_matvec_amd import synth
    st = DecodeStack(synth.GEMMA_MATS + [synth.GEMMA_O], synth.GEMMA_LAYERS, synth.CONFIG_GEMMA_DECODE, 1, copies,
                     dev)
    step_ms, gemv_ms, _, _ = time_decode(st, reps, 10, stream)
    out = {"workload": "ternary batch-1 decode, Gemma-3-1B shapes x26 with o_proj (182 matrices)",
           "gemv_us": us(gemv_ms), "step_us": us(step_ms), "gemv_bytes": st.gemv_bytes(),
           "GB/s": round(st.gemv_bytes() / gemv_ms / 1e6, 1),
           "frac_hbm_peak": round(st.gemv_bytes() / gemv_ms / 1e6 / HBM_PEAK_GBS, 4)}
    del st
    torch.cuda.empty_cache()
    return out


def bench_zero_skip(dev, stream, reps, copies, dense=True):
    """Zero-group skipping: the Gemma step with 80% of the activations' groups of 4
    columns zero, on the dense plan and on the plan that skips 20-column units
    whose activations are all zero."""
    import torch
    from ternary_matvec_amd import qmv, synth
    st = DecodeStack(synth.GEMMA_MATS, synth.GEMMA_LAYERS, synth.CONFIG_GEMMA_DECODE, 1, copies, dev,
                     zero_groups=True)
    zero_units, units = 0, 0
    for v in st.x_host.values():   # 20-column units (4 packed bytes), the last one zero padded
        pad = np.zeros((v.shape[0], (v.shape[1] + 19) // 20 * 20), np.float32)
        pad[:, :v.shape[1]] = v
        u = (pad.reshape(v.shape[0], -1, 20) == 0).all(axis=2)
        zero_units += int(u.sum())
        units += u.size
    skip = st.plan_kind(qmv.QMV_PLAN_GEMV_SKIP_ZERO)
    skip_ms, _ = median_time(lambda i: skip[i % copies].launch(stream), reps, stream)
    out = {"workload": "Gemma-3-1B x26 decode, activations with 80% zero groups of 4 columns",
           "zero_20_column_units": round(zero_units / max(units, 1), 3), "skip_plan_us": us(skip_ms)}
    if dense:
        dense_ms, _ = median_time(lambda i: st.plans[i % copies].launch(stream), reps, stream)
        out["dense_plan_us"] = us(dense_ms)
        out["speedup"] = round(dense_ms / skip_ms, 3)
    del st, skip
    torch.cuda.empty_cache()
    return out


def bench_bitnet(dev, stream, reps, copies, ms_list=(1, 2, 4, 8, 16), dot_compare=(2, 4)):
    """BitNet-b1.58-large shapes x24 (168 matrices) at several tokens per step:
    the default plan's kernel, and the dot-product plan beside the matrix-core
    one."""
    import torch
    from ternary_matvec_amd import qmv, synth
    out = {}
    for m in ms_list:
        st = DecodeStack(synth.BITNET_MATS, synth.BITNET_LAYERS, synth.CONFIG_BITNET, m, copies, dev)
        step_ms, gemv_ms, _, _ = time_decode(st, reps, 5, stream)
        row = {"kernel": route_of(m), "gemv_us": us(gemv_ms), "step_us": us(step_ms),
               "gemv_GB/s": round(st.gemv_bytes() / gemv_ms / 1e6, 1),
               "frac_hbm_peak": round(st.gemv_bytes() / gemv_ms / 1e6 / HBM_PEAK_GBS, 4),
               "weights_per_s": float("%.4g" % (st.weights() / gemv_ms * 1e3)),
               "MAC/s": float("%.4g" % (st.macs() / gemv_ms * 1e3))}
        if m in dot_compare:
            dot = st.plan_kind(qmv.QMV_PLAN_GEMV_DOT)
            dms, _ = median_time(lambda i: dot[i % copies].launch(stream), reps, stream)
            row["dot_plan_us"] = us(dms)
            del dot
        out["m%d" % m] = row
        del st
        torch.cuda.empty_cache()
    return out


def bench_head(dev, stream, reps=50):
    import torch
    from ternary_matvec_amd import qmv, synth
    v, k = synth.HEAD_V, synth.HEAD_K
    w0 = synth.normal_torch(synth.stream_seed(synth.CONFIG_HEAD, 0, 0, synth.TAG_HEAD), (v, k), std=0.02, device=dev)
    copies = [w0.to(torch.bfloat16)]
    del w0
    copies.append(copies[0].clone())
    x = torch.from_numpy(synth.normal(synth.stream_seed(synth.CONFIG_HEAD, 0, 0, synth.TAG_ACT), (k,))).to(dev)
    ws = qmv._alloc_aligned(qmv.qmv_lmhead_workspace_bytes(v, k), dev)
    idx = torch.empty(1, dtype=torch.int32, device=dev)
    mx = torch.empty(1, dtype=torch.float32, device=dev)
    ms, _ = median_time(lambda i: qmv.qmv_lmhead_argmax(copies[i % 2], x, idx=idx, max_logit=mx, workspace=ws,
                                                       stream=stream), reps, stream)
    nbytes = v * k * 2 + 4 * k + 8
    return {"workload": "bf16 output layer 262144x1152 + first-max argmax", "us": us(ms),
            "GB/s": round(nbytes / ms / 1e6, 1), "frac_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
            "idx": int(idx.item())}


def bench_sketch(dev, stream, reps=50, copies=6, tokens=32):
    """The sketch head on the output layer: time per token with the tables
    rotated over `copies` weight/sketch pairs (so they come from HBM, not the
    256 MB last-level cache), the same on one pair (cache-resident), and how
    often it picks the exact argmax: on random hidden states, and on peaked
    ones (x close to one word's row, like a confident model)."""
    import torch
    from ternary_matvec_amd import qmv, synth
    v, k = synth.HEAD_V, synth.HEAD_K
    w0 = synth.normal_torch(synth.stream_seed(synth.CONFIG_HEAD, 0, 0, synth.TAG_HEAD), (v, k), std=0.02, device=dev)
    ws_ = [w0.to(torch.bfloat16)]
    del w0
    for _ in range(copies - 1):
        ws_.append(ws_[0].clone())
    sk = [qmv.qmv_sketch_build(w) for w in ws_]
    torch.cuda.synchronize()
    wsp = qmv.sketch_workspace(v, k, dev)
    xs = [torch.from_numpy(synth.normal(synth.stream_seed(synth.CONFIG_HEAD, 1, t, synth.TAG_ACT), (k,))).to(dev)
          for t in range(tokens)]
    idx = torch.empty(1, dtype=torch.int32, device=dev)
    mx = torch.empty(1, dtype=torch.float32, device=dev)
    nc = torch.empty(1, dtype=torch.int32, device=dev)

    def call(i, n_pairs):
        qmv.qmv_lmhead_sketch_argmax(ws_[i % n_pairs], sk[i % n_pairs], xs[i % tokens], idx=idx, max_logit=mx,
                                     candidates=nc, workspace=wsp, stream=stream)

    ms_hbm, _ = median_time(lambda i: call(i, copies), reps, stream)
    ms_cached, _ = median_time(lambda i: call(i, 1), reps, stream)
    wsl = qmv._alloc_aligned(qmv.qmv_lmhead_workspace_bytes(v, k), dev)
    wf = ws_[0].float()
    rng = np.random.default_rng(5)
    agree = {"random": 0, "peaked": 0}
    ncands = []
    for kind in ("random", "peaked"):
        for t in range(tokens):
            if kind == "random":
                x = xs[t]
            else:
                r = int(rng.integers(0, v))
                x = (8.0 * wf[r] + torch.from_numpy(synth.normal(synth.stream_seed(synth.CONFIG_HEAD, 2, t,
                                                                                   synth.TAG_ACT),
                                                                 (k,))).to(dev) * 0.05).contiguous()
            qmv.qmv_lmhead_sketch_argmax(ws_[0], sk[0], x, idx=idx, max_logit=mx, candidates=nc, workspace=wsp,
                                         stream=stream)
            ie, _, _ = qmv.qmv_lmhead_argmax(ws_[0], x, workspace=wsl, stream=stream)
            torch.cuda.synchronize()
            agree[kind] += int(idx.item() == ie.item())
            ncands.append(int(nc.item()))
    kw = (k + 31) // 32
    cand = float(np.mean(ncands))
    nbytes = 4 * kw * v + 2 * 32 * v + cand * 2 * k + 8 * v + 4 * k
    return {"workload": "sketch head on the bf16 output layer 262144x1152: 32 exact dims + 1-bit groups, "
                        ">=1024 candidates rescored",
            "us": us(ms_hbm), "us_cache_resident": us(ms_cached),
            "weight_copies": copies, "bytes_per_token": int(nbytes), "GB/s": round(nbytes / ms_hbm / 1e6, 1),
            "candidates_mean": round(cand, 1),
            "agrees_with_exact_argmax": {k_: "%d/%d" % (a, tokens) for k_, a in agree.items()}}


def ffn_stack(stack, dev):
    """The decode stack's gate/up/down (copy 0) with RMSNorm weights: the
    feed-forward half of its 26 layers, and a residual stream h."""
    import torch
    from ternary_matvec_amd import qmv, synth
    names = [name for (name, _, _) in stack.mats]
    gi, ui, di = names.index("gate"), names.index("up"), names.index("down")
    nm = len(names)
    hidden, inter = stack.mats[gi][2], stack.mats[gi][1]
    arr = (qmv.qmv_ffn_layer * stack.layers)()
    norms = []
    for layer in range(stack.layers):
        norm = torch.from_numpy(synth.normal(synth.stream_seed(7, layer, 1, synth.TAG_MISC), (hidden,)) * 0.1
                                + 1.0).to(dev)
        norms.append(norm)
        arr[layer].gate = stack.arrays[0][layer * nm + gi].w
        arr[layer].up = stack.arrays[0][layer * nm + ui].w
        arr[layer].down = stack.arrays[0][layer * nm + di].w
        arr[layer].norm = norm.data_ptr()
    h0 = torch.from_numpy(synth.normal(synth.stream_seed(7, 0, 0, synth.TAG_ACT), (hidden,))).to(dev)
    return arr, norms, h0, hidden, inter, (gi, ui, di, nm)


def bench_ffn(stack, dev, stream, reps=50, chain=True):
    """The feed-forward half of the 26 layers for one token, h += down(GLU(gate, up)(RMSNorm(h))):
    as the launch-per-step chain (qmv_rmsnorm_quantize, one grouped qmv_gemv for gate and up,
    qmv_glu_quantize, qmv_gemv for down, an fp32 add: 130 launches), eager and as a graph
    replay, and as one persistent qmv_ffn_decode launch; with the fused steps alone."""
    import torch
    from ternary_matvec_amd import qmv, synth
    arr, norms, h0, hidden, inter, (gi, ui, di, nm) = ffn_stack(stack, dev)
    x8a = torch.empty((1, hidden), dtype=torch.int8, device=dev)
    sxa = torch.empty(1, dtype=torch.float32, device=dev)
    yg = torch.empty((1, inter), dtype=torch.float32, device=dev)
    yu = torch.empty((1, inter), dtype=torch.float32, device=dev)
    x8b = torch.empty((1, inter), dtype=torch.int8, device=dev)
    sxb = torch.empty(1, dtype=torch.float32, device=dev)
    yd = torch.empty((1, hidden), dtype=torch.float32, device=dev)
    h = h0.clone()

    def prob(w, x8, sx, y):
        p = qmv.qmv_problem()
        p.w = w
        p.x8, p.sx, p.m, p.y, p.acc = x8.data_ptr(), sx.data_ptr(), 1, y.data_ptr(), None
        return p

    layers = []
    for layer in range(stack.layers):
        gu = (qmv.qmv_problem * 2)(prob(arr[layer].gate, x8a, sxa, yg), prob(arr[layer].up, x8a, sxa, yu))
        dn = (qmv.qmv_problem * 1)(prob(arr[layer].down, x8b, sxb, yd))
        layers.append((qmv.gemv_plan(gu, stream=stream), qmv.gemv_plan(dn, stream=stream), norms[layer]))
    torch.cuda.synchronize()

    def token(s):
        for gu, dn, norm in layers:
            qmv.qmv_rmsnorm_quantize(h.view(1, hidden), norm, 1e-6, x8=x8a, sx=sxa, stream=s)
            gu.launch(s)
            qmv.qmv_glu_quantize(yg, yu, qmv.QMV_ACT_GELU_TANH, x8=x8b, sx=sxb, stream=s)
            dn.launch(s)
            with torch.cuda.stream(s):
                h.add_(yd.view(hidden))

    ws = qmv.ffn_workspace(hidden, inter, dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {}
    if chain:
        chain_ms, _ = median_time(lambda i: token(stream), reps, stream)
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                token(cap)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        graph_ms, _ = median_time(lambda i: graph.replay(), reps, stream)
        # the persistent launch against the chain on one token
        h.copy_(h0)
        token(stream)
        ref = h.clone()
        h.copy_(h0)
        qmv.qmv_ffn_decode(arr, h, eps=1e-6, act=qmv.QMV_ACT_GELU_TANH, workspace=ws, status=status, stream=stream)
        torch.cuda.synchronize()
        res = {"chain_us_per_token": us(chain_ms), "chain_graph_replay_us_per_token": us(graph_ms),
               "chain_launches_per_token": 5 * stack.layers,
               "persistent_equals_chain": bool(torch.equal(h, ref)) and int(status.item()) == 0}
    pers_ms, pers_all = median_time(lambda i: qmv.qmv_ffn_decode(arr, h, eps=1e-6, act=qmv.QMV_ACT_GELU_TANH,
                                                                 workspace=ws, status=status, stream=stream),
                                    reps, stream)
    # where a persistent launch spends a layer (its own trace, medians over layers 1..25)
    grid = qmv.qmv_ffn_grid()
    S = qmv.QMV_FFN_TRACE_STAMPS
    tr = torch.zeros((grid, 1 + S * stack.layers), dtype=torch.int64, device=dev)
    qmv.qmv_ffn_decode(arr, h, eps=1e-6, act=qmv.QMV_ACT_GELU_TANH, workspace=ws, status=status, trace=tr,
                       stream=stream)
    torch.cuda.synchronize()
    t = tr.cpu().numpy().astype(np.float64)[:, 1:].reshape(grid, stack.layers, S) * 0.01   # us
    gu = t[:min(grid, (inter + 31) // 32)]
    dn = t[t[:, 0, 9] > 0]

    def med(x, a, b):
        return round(float(np.median(x[:, 1:, b] - x[:, 1:, a])), 2)

    breakdown = {"gate_up_path_us": {"rmsnorm_and_codes": med(gu, 1, 4), "gate_up_dots_and_glu": med(gu, 4, 5)},
                 "down_path_us": {"inputs_to_dots": med(dn, 6, 8), "atomics_acknowledged": med(dn, 8, 9)},
                 "exchange_us": {
                     "down_done_to_gate_up_inputs": round(float(np.median(
                         [gu[:, l, 1].min() - dn[:, l - 1, 9].max() for l in range(1, stack.layers)])), 2),
                     "gate_up_done_to_down_inputs": round(float(np.median(
                         [dn[:, l, 6].min() - gu[:, l, 5].max() for l in range(1, stack.layers)])), 2)},
                 "per_layer_us": round(float((t[:, -1, 10].max() - t[:, 0, 10].max()) / (stack.layers - 1)), 2)}
    wbytes = stack.layers * sum(n * ((k + 4) // 5) for (name, n, k) in stack.mats if name in ("gate", "up", "down"))
    out = {"workload": "Gemma-3-1B feed-forward half x26 layers, one token: RMSNorm->int8, gate+up, "
                       "GeLU(gate)*up->int8, down, residual add",
           "weight_bytes": wbytes}
    out.update(res)
    out.update({"persistent_us_per_token": us(pers_ms), "persistent_GB/s": round(wbytes / pers_ms / 1e6, 1),
                "persistent_grid": grid, "persistent_breakdown": breakdown})
    if chain:
        out["speedup_vs_chain"] = round(res["chain_us_per_token"] / us(pers_ms), 2)
        r1, _ = median_time(lambda i: qmv.qmv_rmsnorm_quantize(h.view(1, hidden), norms[0], 1e-6, x8=x8a, sx=sxa,
                                                               stream=stream), 200, stream)
        g1, _ = median_time(lambda i: qmv.qmv_glu_quantize(yg, yu, qmv.QMV_ACT_GELU_TANH, x8=x8b, sx=sxb,
                                                           stream=stream), 200, stream)
        out["rmsnorm_quantize_us_1x%d" % hidden] = us(r1)
        out["glu_quantize_us_1x%d" % inter] = us(g1)
    return out


def bench_int8(dev, stream, reps=2000):
    import torch
    from ternary_matvec_amd import qmv, synth
    n, k = synth.INT8_N, synth.INT8_K
    w = torch.from_numpy(synth.normal(synth.stream_seed(synth.CONFIG_INT8, 0, 0, synth.TAG_WEIGHT), (n, k),
                                      std=0.02)).to(dev)
    x = torch.from_numpy(synth.normal(synth.stream_seed(synth.CONFIG_INT8, 0, 0, synth.TAG_ACT), (1, k))).to(dev)
    pw = qmv.qmv_pack_int8(w)
    x8, sx = qmv.qmv_quantize_act(x)
    y = torch.empty((1, n), dtype=torch.float32, device=dev)   # owned here for as long as the plan runs
    prob = qmv.Problem(pw, x8, sx, y=y)
    plan = qmv.gemv_plan([prob])
    torch.cuda.synchronize()

    def both(i):
        qmv.qmv_quantize_act(x, x8=x8, sx=sx, stream=stream)
        plan.launch(stream)

    ms, _ = median_time(both, reps, stream)
    gms, _ = median_time(lambda i: plan.launch(stream), reps, stream)
    nbytes = n * k + 5 * k + 4 * n + 8
    return {"workload": "int8 per-tensor GEMV 768x288, batch 1", "us_per_call_quantise_and_gemv": us(ms),
            "us_per_gemv": us(gms), "GB/s": round(nbytes / ms / 1e6, 2)}


def bench_groupscale(dev, stream, reps=100, copies=2):
    """Gemma-3-1B shapes x26 with int8 weights in groups of 128 and activation
    scales per 32 columns, batch 1: one grouped qmv_gemv launch of 156 problems."""
    import torch
    from ternary_matvec_amd import qmv, synth
    cfg = synth.CONFIG_GEMMA_DECODE
    specs = [(layer, mid, n, k) for layer in range(synth.GEMMA_LAYERS) for mid, (_, n, k) in enumerate(synth.GEMMA_MATS)]
    wbytes = sum(qmv.qmv_packed_bytes(qmv.QMV_W_INT8_G128, n, k) for (_, _, n, k) in specs)
    nscale = sum(n * ((k + 127) // 128) for (_, _, n, k) in specs)
    pools = [qmv._alloc_aligned(wbytes, dev, 256) for _ in range(copies)]
    spool = [torch.empty(nscale, dtype=torch.float32, device=dev) for _ in range(copies)]
    descs, off, soff = [], 0, 0
    for (layer, mid, n, k) in specs:
        nb = qmv.qmv_packed_bytes(qmv.QMV_W_INT8_G128, n, k)
        ns = n * ((k + 127) // 128)
        w = synth.normal_torch(synth.stream_seed(cfg, layer, mid, synth.TAG_WEIGHT), (n, k), std=0.02, device=dev)
        for c in range(copies):   # packed per copy: no device copy larger than the counter calibration's
            qmv.qmv_pack_int8_grouped(w, packed=pools[c][off:off + nb], scales=spool[c][soff:soff + ns])
        descs.append((n, k, off, nb, soff, ns))
        off += nb
        soff += ns
        del w
    torch.cuda.synchronize()
    xs = [torch.from_numpy(synth.normal(synth.stream_seed(cfg, layer, mid, synth.TAG_ACT), (1, k))).to(dev)
          for (layer, mid, n, k) in specs]
    acts = [qmv.qmv_quantize_act_grouped(x) for x in xs]
    ys = [torch.empty((1, n), dtype=torch.float32, device=dev) for (_, _, n, _) in specs]
    plans = []
    for c in range(copies):
        probs = []
        for i, (n, k, o, nb, so, ns) in enumerate(descs):
            wc = qmv.Weight(qmv.qmv_weight(qmv.QMV_W_INT8_G128, 0, n, k, pools[c][o:].data_ptr(),
                                           spool[c][so:].data_ptr()), pools[c][o:o + nb], spool[c][so:so + ns])
            probs.append(qmv.Problem(wc, acts[i][0], acts[i][1], y=ys[i]))
        plans.append(qmv.gemv_plan(qmv.problem_array(probs)))
    torch.cuda.synchronize()
    ms, _ = median_time(lambda i: plans[i % copies].launch(stream), reps, stream)
    nbytes = wbytes + 4 * nscale + sum(k + 4 * ((k + 31) // 32) + 4 * n for (_, _, n, k) in specs)
    out = {"workload": "int8 weights in groups of 128 columns, activation scales per 32, Gemma-3-1B shapes x26 "
                       "(156 matrices), batch 1, one grouped launch", "weight_copies": copies,
           "bytes_per_launch": nbytes, "us_per_launch": us(ms), "GB/s": round(nbytes / ms / 1e6, 1),
           "frac_of_8TBps": round(nbytes / ms / 8e6, 3)}
    del pools, spool, plans
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# CPU oracle baselines (bounded samples; the oracle as it stands)
# ---------------------------------------------------------------------------

def _cpu_inputs(specs, config_id, x_of, dev):
    from ternary_matvec_amd import synth
    out = []
    for (lay, mid, name, n, k, slot) in specs:
        t = synth.trits_torch(synth.stream_seed(config_id, lay, mid, synth.TAG_WEIGHT), (n, k),
                              device=dev).cpu().numpy()
        s = synth.ternary_scale(synth.stream_seed(config_id, lay, mid, synth.TAG_SCALE))
        out.append((t, x_of(lay, mid, n, k, slot), np.float32(s)))
    return out


def _oracle_pass(inputs, threads):
    import oracle
    for (t, x, s) in inputs:
        q, sx = oracle.quantize_rows(x)
        acc = oracle.matmul_int(q, t, threads=threads)
        oracle.dequant(acc, sx, s)


def _median3(fn):
    vals = []
    for _ in range(3):
        t0 = time.perf_counter()
        fn()
        vals.append(time.perf_counter() - t0)
    return float(np.median(vals))


def cpu_baseline(stack, target_s, dev):
    """C2 on the oracle (per-token quantise, exact integer matmul from trits,
    dequantise) over whole steps of the same workload, repeated until about
    `target_s` seconds of CPU work."""
    import oracle
    threads = oracle.max_threads()
    inputs = _cpu_inputs(stack.specs, stack.config_id,
                         lambda lay, mid, n, k, slot: stack.x_host[k][slot * stack.m:(slot + 1) * stack.m], dev)
    elapsed, passes = 0.0, 0
    while passes == 0 or elapsed < target_s:
        t0 = time.perf_counter()
        _oracle_pass(inputs, threads)
        elapsed += time.perf_counter() - t0
        passes += 1
    value = stack.step_bytes() * passes / elapsed / 1e9
    return {"value": round(value, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d full step(s) of the same workload (%d matrices, batch %d): per-token quantise, exact "
                      "int matmul from unpacked trits, dequantise; %.1f s on %d threads, %.1f ms per step"
                      % (passes, len(stack.specs), stack.m, elapsed, threads, elapsed / passes * 1e3)}


def cpu_baselines(stack, dev):
    """The oracle on the other configurations (median of 3 where a sample is
    under a few seconds): C1 in full, C3 as one layer's 6 matrices x 512 tokens
    (x26 reported as extrapolated), C4 in full, C5 one full step at 1, 4 and 16
    tokens, and C2's first layer on one thread."""
    import oracle
    import torch
    from ternary_matvec_amd import synth
    threads = oracle.max_threads()
    out = {"cores": threads, "kind": "oracle"}
    # C1: int8 768x288
    n, k = synth.INT8_N, synth.INT8_K
    w = synth.normal(synth.stream_seed(synth.CONFIG_INT8, 0, 0, synth.TAG_WEIGHT), (n, k), std=0.02)
    x = synth.normal(synth.stream_seed(synth.CONFIG_INT8, 0, 0, synth.TAG_ACT), (1, k))
    w8, sw = oracle.quantize_tensor(w)

    def c1():
        for _ in range(200):
            q, sx = oracle.quantize_rows(x)
            acc = oracle.matmul_int(q, w8, threads=threads)
            oracle.dequant(acc, sx, sw)
    s = _median3(c1) / 200
    out["C1_int8_768x288"] = {"us_per_call": round(s * 1e6, 1), "GB/s": round((n * k + 5 * k + 4 * n + 8) / s / 1e9, 4)}
    # C3: layer 0's six matrices at 512 tokens
    m = 512
    spec0 = stack.specs[:len(stack.mats)]
    xs = {}
    for (lay, mid, name, nn, kk, slot) in spec0:
        xs[(lay, mid)] = synth.normal_torch(synth.stream_seed(synth.CONFIG_GEMMA_PREFILL, lay, mid, synth.TAG_ACT),
                                            (m, kk), device=dev).cpu().numpy()
    inputs = _cpu_inputs(spec0, stack.config_id, lambda lay, mid, nn, kk, slot: xs[(lay, mid)], dev)
    s = _median3(lambda: _oracle_pass(inputs, threads))
    ops = 2 * m * sum(nn * kk for (_, _, _, nn, kk, _) in spec0)
    out["C3_prefill_512"] = {"one_layer_s": round(s, 3), "x26_extrapolated_s": round(26 * s, 2),
                             "TOPS": round(ops / s / 1e12, 4), "sample": "layer 0's 6 matrices x 512 tokens"}
    del inputs, xs
    # C4: the bf16 output layer, exact fp64 scores and first max
    v, kh = synth.HEAD_V, synth.HEAD_K
    wh = synth.normal_torch(synth.stream_seed(synth.CONFIG_HEAD, 0, 0, synth.TAG_HEAD), (v, kh), std=0.02,
                            device=dev).to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    xh = synth.normal(synth.stream_seed(synth.CONFIG_HEAD, 0, 0, synth.TAG_ACT), (kh,))
    s = _median3(lambda: oracle.lmhead(wh, xh, threads=threads))
    out["C4_lmhead_262144x1152"] = {"ms": round(s * 1e3, 1), "GB/s": round((v * kh * 2 + 4 * kh + 8) / s / 1e9, 3)}
    del wh
    # C5: BitNet-large, one full step at 1, 4, 16 tokens
    c5 = {}
    specs5 = []
    rows = {}
    for layer in range(synth.BITNET_LAYERS):
        for mid, (name, nn, kk) in enumerate(synth.BITNET_MATS):
            specs5.append((layer, mid, name, nn, kk, 0))
    tr5 = _cpu_inputs(specs5, synth.CONFIG_BITNET, lambda *a: None, dev)
    for mm in (1, 4, 16):
        inp = []
        for (lay, mid, name, nn, kk, _), (t, _, sc) in zip(specs5, tr5):
            xk = rows.setdefault((lay, mid, mm), synth.normal(synth.stream_seed(synth.CONFIG_BITNET, lay, mid,
                                                                                synth.TAG_ACT), (mm, kk)))
            inp.append((t, xk, sc))
        s = _median3(lambda: _oracle_pass(inp, threads))
        wbytes = sum(nn * ((kk + 4) // 5) for (_, _, _, nn, kk, _) in specs5)
        c5["m%d" % mm] = {"ms_per_step": round(s * 1e3, 1), "GB/s": round(wbytes / s / 1e9, 4),
                          "MAC/s": float("%.4g" % (mm * sum(nn * kk for (_, _, _, nn, kk, _) in specs5) / s))}
    out["C5_bitnet_large_x24"] = c5
    del tr5
    # C2's first layer on one thread
    inputs = _cpu_inputs(stack.specs[:len(stack.mats)], stack.config_id,
                         lambda lay, mid, nn, kk, slot: stack.x_host[kk][slot * stack.m:(slot + 1) * stack.m], dev)
    s = _median3(lambda: _oracle_pass(inputs, 1))
    nb = sum(nn * ((kk + 4) // 5) + 6 * kk + 4 * nn + 8 for (_, _, _, nn, kk, _) in stack.specs[:len(stack.mats)])
    out["C2_one_layer_1_thread"] = {"ms": round(s * 1e3, 2), "GB/s": round(nb / s / 1e9, 4)}
    return out


# ---------------------------------------------------------------------------

def main():
    global WARM_MS
    args = parse()
    WARM_MS = max(0.0, args.warm_ms)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    from ternary_matvec_amd import qmv, synth
    qmv.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    reps = max(100, args.steps)

    log("building the Gemma-shaped decode stack (26 layers x 6 matrices, %d copies)" % args.copies)
    t0 = time.perf_counter()
    stack = DecodeStack(synth.GEMMA_MATS, synth.GEMMA_LAYERS, synth.CONFIG_GEMMA_DECODE, 1, args.copies, dev)
    log("stack ready in %.1f s: %.1f MB packed per copy" % (time.perf_counter() - t0, stack.packed_bytes / 1e6))

    step_ms, gemv_ms, step_all, gemv_all = time_decode(stack, reps, args.warmup, stream)
    log("step %.2f us, grouped GEMV %.2f us (median of %d x %d back-to-back)" %
        (step_ms * 1e3, gemv_ms * 1e3, N_REP, reps))
    ceiling_gbs, ceiling_ms = time_read_ceiling(stack, reps, stream)
    log("plain read of the weight copies: %.1f GB/s" % ceiling_gbs)

    step_bytes = stack.step_bytes()
    gemv_bytes = stack.gemv_bytes()
    value = step_bytes / step_ms / 1e6          # GB/s
    achieved = gemv_bytes / gemv_ms / 1e6
    result = {
        "metric": "batch-1 ternary GEMV achieved HBM GB/s (% of peak) + prefill int8 TOPS",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x trit -> int32, fp32 scales",
        "data": "synthetic (splitmix64 seed 42: trits P(-1,0,1)=(.3,.4,.3), x ~ N(0,1))",
        "config": {"workload": "ternary batch-1 decode, Gemma-3-1B shapes x26 layers (156 matrices: q 1024x1152, "
                               "k/v 256x1152, gate/up 6912x1152, down 1152x6912), 5 trits/byte",
                   "tokens": 1, "matrices": len(stack.specs), "weight_copies": args.copies,
                   "step": "qmv_quantize_act_many (both widths, one launch) + one grouped qmv_gemv plan launch",
                   "step_bytes": step_bytes, "weights_per_step": stack.weights(),
                   "weights_per_s": float("%.4g" % (stack.weights() / step_ms * 1e3)),
                   "timing": "median of %d repetitions of %d back-to-back steps, HIP events on the launch stream"
                             % (N_REP, reps),
                   "step_us_reps": [us(v) for v in step_all], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "k_gemv_stream<1,1,false> (grouped ternary GEMV)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": gemv_traffic(),
                     "bytes_per_launch": gemv_bytes, "launch_us": us(gemv_ms),
                     "launch_us_reps": [us(v) for v in gemv_all],
                     "launch_timing": "median of %d repetitions of %d back-to-back launches, HIP events on the "
                                      "launch stream" % (N_REP, reps),
                     "measured_read_ceiling": round(ceiling_gbs, 1),
                     "frac_of_measured_ceiling": round(achieved / ceiling_gbs, 4),
                     "ceiling_kernel": "qmv_read_probe: one non-temporal 16-byte-load read of the same weight copies "
                                       "(%.1f MB in %.2f us)" % (stack.pool[0].numel() / 1e6, ceiling_ms * 1e3)},
    }
    # the decode rows beside the headline: the same plan launches as the
    # headline's, on the "+o_proj" stack and on the BitNet-large shapes (in the
    # profile set only the matrix-core rows, so that every kernel name in a
    # profile comes from one workload)
    rows = ((("bitnet_decode", lambda: bench_bitnet(dev, stream, reps, min(args.copies, 8), ms_list=(4, 16),
                                                    dot_compare=())),) if args.profile_set else
            (("decode_o_proj", lambda: bench_o_proj(dev, stream, reps, args.copies)),
             ("bitnet_decode", lambda: bench_bitnet(dev, stream, reps, min(args.copies, 8), ms_list=(1, 4, 16),
                                                    dot_compare=(4, 16)))))
    for name, fn in rows:
        log(name)
        result[name] = fn()
        torch.cuda.synchronize()
    for key, r in result["bitnet_decode"].items():
        log("bitnet %s: %.1f us (%s)" % (key, r["gemv_us"], r["kernel"]))
    log("prefill (512 tokens)")
    result["prefill"] = bench_prefill(stack, dev, stream)
    log("prefill %.1f us, %.1f TOPS" % (result["prefill"]["prefill_us"], result["prefill"]["TOPS"]))
    # opt-in extras (in the profile set, the forms the profiles describe)
    ps = args.profile_set
    runs = {"decode_copies_sweep": lambda: copies_sweep(stack, reps, stream),
            "decode_chained": lambda: chained(stack, 20, stream),
            "quantize_step": lambda: {"us": us(median_time(lambda i: qmv.qmv_quantize_act_many(
                stack.acts, stream=stream), reps, stream)[0]), "bytes": stack.quant_bytes()},
            "host_overhead": lambda: host_overhead(stack, stream),
            "ffn": lambda: bench_ffn(stack, dev, stream, chain=not ps),
            "zero_skip": lambda: bench_zero_skip(dev, stream, reps, min(args.copies, 4), dense=not ps),
            "lmhead": lambda: bench_head(dev, stream),
            "lmhead_sketch": lambda: bench_sketch(dev, stream),
            "int8_gemv": lambda: bench_int8(dev, stream),
            "groupscale_decode": lambda: bench_groupscale(dev, stream),
            "bitnet_decode_all": lambda: bench_bitnet(dev, stream, reps, min(args.copies, 8),
                                                      ms_list=(1, 2, 4, 8, 16), dot_compare=(2, 4, 8, 16))}
    extras = {}
    for name in args.extras:
        log(name)
        extras[name] = runs[name]()   # an error ends the run: nothing is reported past a failed launch
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if "us" in extras.get("lmhead", {}) and "us" in extras.get("lmhead_sketch", {}):
        extras["lmhead_sketch"]["speedup_vs_full_head"] = round(extras["lmhead"]["us"] /
                                                                extras["lmhead_sketch"]["us"], 2)
    if extras:
        result["extras"] = extras
    if args.copy_probe_mb:
        nbytes = args.copy_probe_mb << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = nbytes
        del src, dst
    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        try:
            result["cpu_baseline"] = cpu_baseline(stack, args.cpu_seconds, dev)
        except Exception as e:
            result["cpu_baseline"] = {"error": repr(e)}
        if not args.profile_set:
            log("CPU oracle on the other configurations")
            try:
                result["cpu_baselines"] = cpu_baselines(stack, dev)
            except Exception as e:
                result["cpu_baselines"] = {"error": repr(e)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
