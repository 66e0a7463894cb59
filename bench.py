"""Benchmark of the quantized matvec hot path on one MI355X.

Headline workload: batch-1 ternary decode over Gemma-3-1B-shaped weights,
26 layers x {q, k, v, gate, up, down} = 156 matrices, trits iid with
P(-1, 0, +1) = (0.3, 0.4, 0.3), one scale per matrix, x ~ N(0, 1).  One step:
  qmv_quantize_act_many on the 130 activation rows of K = 1152 and the 26 rows
  of K = 6912 (one launch), then one grouped qmv_gemv over the 156 problems.
Weights rotate over several full copies so the 256 MB Infinity Cache cannot
hold the working set.  `value` = algorithmic bytes per step / step time.

Also reported (not the headline): 512-token prefill through qmv_gemm_prefill
(int8 TOPS), the 262144 x 1152 bf16 output layer with greedy argmax (GB/s),
the 768 x 288 int8 GEMV (us/call), BitNet-b1.58-large-shaped decode at 1, 4 and
16 tokens, and the CPU oracle timed on the host's cores on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, datasheet
GEMV_SOURCES = ("k_gemv_stream.hip", "unpack.hpp", "qmv_internal.hpp")
GEMV_COUNTERS = os.path.join(ROOT, "profiles", "k_gemv_stream_counters.json")
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA, datasheet


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=8, help="weight copies rotated to defeat the MALL")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="headline workload only")
    ap.add_argument("--profile-set", action="store_true",
                    help="only the launches the kernel profiles describe: decode steps, full prefill passes, "
                         "the output layer, the sketch head and the group-scaled decode (no sweeps, chained, "
                         "per-matrix, int8 or BitNet launches)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-oracle time")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB five times: the "
                         "known-size kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters "
                         "(1024 makes it the largest copy of the run)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# Workload construction
# ---------------------------------------------------------------------------

class DecodeStack:
    """A stack of ternary matrices packed on the GPU, with its activations."""

    def __init__(self, mats, layers, config_id, m, copies, dev):
        import torch
        from ternary_matvec_amd import qmv, synth
        self.mats, self.layers, self.m, self.copies = mats, layers, m, copies
        self.config_id = config_id
        self.weights = []          # per (layer, mid): Weight of copy 0
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
            xs = [synth.normal(synth.stream_seed(config_id, layer, mid, synth.TAG_ACT), (m, kk))
                  for (layer, mid, _, _, kk, _) in self.specs if kk == k]
            self.x_host[k] = np.concatenate(xs, axis=0)
            self.x[k] = torch.from_numpy(self.x_host[k]).to(dev)
        self.x8, self.sx = {}, {}
        for k in ks:
            self.x8[k] = torch.empty(self.x[k].shape, dtype=torch.int8, device=dev)
            self.sx[k] = torch.empty(self.x[k].shape[0], dtype=torch.float32, device=dev)
        # every width's activations quantised by one launch
        self.acts = qmv.act_array([(self.x[k], self.x8[k], self.sx[k]) for k in ks])
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
        # one problem list (and one uploaded table) per copy
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

    # algorithmic bytes ---------------------------------------------------------
    def weight_bytes(self):
        return sum(n * ((k + 4) // 5) for (_, _, _, n, k, _) in self.specs)

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


def time_decode(stack, steps, warmup, stream):
    """Whole steps (quantise + grouped GEMV): K steps timed between two events
    with nothing else in the stream, then K more with the GEMV launch of every
    step bracketed by its own pair of events (its duration; event records between
    launches add a few microseconds of their own, so they stay out of the step
    time)."""
    import torch
    from ternary_matvec_amd import qmv

    def step(i, ev=None):
        qmv.qmv_quantize_act_many(stack.acts, stream=stream)
        c = i % stack.copies
        if ev is not None:
            ev[0].record(stream)
        stack.plans[c].launch(stream)
        if ev is not None:
            ev[1].record(stream)

    for i in range(warmup):
        step(i)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t0.elapsed_time(t1) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    gemv_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    return step_ms, gemv_ms, wall


def time_gemv_only(stack, steps, warmup, stream):
    """Back-to-back grouped GEMV launches (no quantisation), events around the loop."""
    import torch
    from ternary_matvec_amd import qmv
    for i in range(warmup):
        stack.plans[i % stack.copies].launch(stream)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        stack.plans[i % stack.copies].launch(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_read_ceiling(stack, reps, stream):
    """The plain-read yardstick (qmv_read_probe) over the same weight copies, rotated
    like the GEMV's: the HBM read rate this machine reaches on these buffers."""
    import torch
    from ternary_matvec_amd import qmv
    out = torch.zeros(1, dtype=torch.int32, device=stack.pool[0].device)
    for c in range(stack.copies):
        qmv.qmv_read_probe(stack.pool[c], out, stream=stream)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(reps):
        qmv.qmv_read_probe(stack.pool[i % stack.copies], out, stream=stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    return stack.pool[0].numel() / ms / 1e6, ms


def copies_sweep(stack, steps, stream):
    """GEMV GB/s with the weights rotated over C = 1, 2, 4, 8 copies: the rate must be
    flat once the rotating set (C x 137.5 MB) is well past the 256 MB Infinity Cache."""
    import torch
    from ternary_matvec_amd import qmv
    out = {}
    for c_count in (1, 2, 4, 8):
        if c_count > stack.copies:
            break
        for i in range(10):
            stack.plans[i % c_count].launch(stream)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(steps):
            stack.plans[i % c_count].launch(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        out["C%d" % c_count] = {"gemv_us": round(ms * 1e3, 2), "GB/s": round(stack.gemv_bytes() / ms / 1e6, 1)}
    return out


def chained(stack, steps, stream, copies=4):
    """The step as stream-ordered launches instead of one grouped launch: 156 (one per
    matrix) or 78 (q/k/v and gate/up grouped per layer, down alone)."""
    import ctypes
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
        for i in range(3):
            step(i)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(steps):
            step(i)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        out["launches_%s" % name] = {"step_us": round(ms * 1e3, 1),
                                     "GB/s": round(stack.gemv_bytes() / ms / 1e6, 1)}
    return out


def time_quantize(stack, steps, stream):
    """The step's quantisation alone: the one qmv_quantize_act_many launch, and
    for comparison one qmv_quantize_act call per width."""
    import torch
    from ternary_matvec_amd import qmv

    def timed(fn):
        for _ in range(5):
            fn()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(steps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def per_width():
        for k in stack.x:
            qmv.qmv_quantize_act(stack.x[k], x8=stack.x8[k], sx=stack.sx[k], stream=stream)

    ms = timed(lambda: qmv.qmv_quantize_act_many(stack.acts, stream=stream))
    ms_w = timed(per_width)
    return {"us": round(ms * 1e3, 2), "GB/s": round(stack.quant_bytes() / ms / 1e6, 1),
            "us_one_call_per_width": round(ms_w * 1e3, 2)}


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def cpu_baseline(stack, target_s, dev):
    """The oracle (per-token quantise, exact integer matmul from trits,
    dequantise) over whole steps of the same workload, repeated until about
    `target_s` seconds of CPU work."""
    import oracle
    from ternary_matvec_amd import synth
    threads = oracle.max_threads()
    inputs = []
    for (lay, mid, name, n, k, slot) in stack.specs:
        t = synth.trits_torch(synth.stream_seed(stack.config_id, lay, mid, synth.TAG_WEIGHT), (n, k),
                              device=dev).cpu().numpy()
        s = synth.ternary_scale(synth.stream_seed(stack.config_id, lay, mid, synth.TAG_SCALE))
        x = stack.x_host[k][slot * stack.m:(slot + 1) * stack.m]
        inputs.append((t, x, np.float32(s)))
    elapsed, passes = 0.0, 0
    while passes == 0 or elapsed < target_s:
        t0 = time.perf_counter()
        for (t, x, s) in inputs:
            q, sx = oracle.quantize_rows(x)
            acc = oracle.matmul_int(q, t, threads=threads)
            oracle.dequant(acc, sx, s)
        elapsed += time.perf_counter() - t0
        passes += 1
    value = stack.step_bytes() * passes / elapsed / 1e9
    return {"value": round(value, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d full step(s) of the same workload (%d matrices, batch %d): per-token quantise, exact "
                      "int matmul from unpacked trits, dequantise; %.1f s on %d threads"
                      % (passes, len(stack.specs), stack.m, elapsed, threads)}


def cpu_single_thread(stack, target_s, dev):
    """The oracle on one thread over one layer's 6 matrices (repeated to about
    `target_s` seconds), in GB/s of that layer's step bytes."""
    import oracle
    from ternary_matvec_amd import synth
    per_layer = len(stack.mats)
    inputs, nbytes = [], 0
    for (lay, mid, name, n, k, slot) in stack.specs[:per_layer]:
        t = synth.trits_torch(synth.stream_seed(stack.config_id, lay, mid, synth.TAG_WEIGHT), (n, k),
                              device=dev).cpu().numpy()
        s = synth.ternary_scale(synth.stream_seed(stack.config_id, lay, mid, synth.TAG_SCALE))
        x = stack.x_host[k][slot * stack.m:(slot + 1) * stack.m]
        inputs.append((t, x, np.float32(s)))
        m = stack.m
        nbytes += n * ((k + 4) // 5) + m * k + 4 * m * n + 4 + 4 * m + 5 * m * k + 4 * m
    elapsed, passes = 0.0, 0
    while passes == 0 or elapsed < target_s:
        t0 = time.perf_counter()
        for (t, x, s) in inputs:
            q, sx = oracle.quantize_rows(x)
            acc = oracle.matmul_int(q, t, threads=1)
            oracle.dequant(acc, sx, s)
        elapsed += time.perf_counter() - t0
        passes += 1
    return {"value": round(nbytes * passes / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1,
            "sample": "%d pass(es) over layer 0's 6 matrices, %.1f s" % (passes, elapsed)}


# ---------------------------------------------------------------------------
# Extras
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
        torch.cuda.synchronize()

    def ops(self):
        return 2 * sum(self.m * n * k for (_, _, _, n, k, _) in self.stack.specs)

    def bytes(self):
        """Algorithmic bytes of one pass: packed weights, int8 activations in, fp32 outputs out."""
        m = self.m
        return sum(n * ((k + 4) // 5) + m * k + 4 * m * n + 4 + 4 * m for (_, _, _, n, k, _) in self.stack.specs)


def time_prefill(ps, steps, warmup, stream):
    import torch
    from ternary_matvec_amd import qmv

    def step(ev=None):
        qmv.qmv_quantize_act_many(ps.acts, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        ps.plan.launch(stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, float(np.mean([a.elapsed_time(b) for a, b in evs]))


def prefill_per_matrix(ps, stream, reps=10):
    """One grouped launch per matrix kind (its 26 layers), timed alone."""
    import torch
    from ternary_matvec_amd import qmv
    specs = ps.stack.specs
    out = {}
    for mid, (name, n, k) in enumerate(ps.stack.mats):
        idx = [i for i, sp in enumerate(specs) if sp[1] == mid]
        sub = (qmv.qmv_problem * len(idx))(*[ps.arr[i] for i in idx])
        plan = qmv.prefill_plan(sub, stream=stream)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(reps):
            plan.launch(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        ops = 2 * ps.m * n * k * len(idx)
        out[name] = {"shape": "%dx%d" % (n, k), "matrices": len(idx), "us": round(ms * 1e3, 1),
                     "TOPS": round(ops / ms / 1e9, 1)}
    return out


def bench_prefill(stack, dev, stream, steps=20, warmup=3, per_matrix=False):
    import torch
    ps = PrefillStack(stack, 512, dev)
    step_ms, kern_ms = time_prefill(ps, steps, warmup, stream)
    tops = ps.ops() / kern_ms / 1e9
    out = {"workload": "ternary prefill, 512 tokens x Gemma-3-1B shapes x26 layers (156 matrices)",
           "kernel": "k_prefill (v_mfma_i32_32x32x32_i8)", "prefill_us": round(kern_ms * 1e3, 1),
           "step_us": round(step_ms * 1e3, 1), "TOPS": round(tops, 1),
           "frac_int8_mfma_peak": round(tops / INT8_PEAK_TOPS, 4),
           "GB/s": round(ps.bytes() / kern_ms / 1e6, 1), "ops_per_pass": ps.ops(), "bytes_per_pass": ps.bytes()}
    if per_matrix:
        out["per_matrix"] = prefill_per_matrix(ps, stream)
    del ps
    torch.cuda.empty_cache()
    return out


def bench_head(dev, stream, reps=50):
    import torch
    from ternary_matvec_amd import qmv, synth
    v, k = synth.HEAD_V, synth.HEAD_K
    w0 = synth.normal_torch(synth.stream_seed(3, 0, 0, synth.TAG_HEAD), (v, k), std=0.02, device=dev)
    copies = [w0.to(torch.bfloat16)]
    del w0
    copies.append(copies[0].clone())
    x = torch.from_numpy(synth.normal(synth.stream_seed(3, 0, 0, synth.TAG_ACT), (k,))).to(dev)
    ws = qmv._alloc_aligned(qmv.qmv_lmhead_workspace_bytes(v, k), dev)
    idx = torch.empty(1, dtype=torch.int32, device=dev)
    mx = torch.empty(1, dtype=torch.float32, device=dev)
    for i in range(5):
        qmv.qmv_lmhead_argmax(copies[i % 2], x, idx=idx, max_logit=mx, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(reps):
        qmv.qmv_lmhead_argmax(copies[i % 2], x, idx=idx, max_logit=mx, workspace=ws, stream=stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    nbytes = v * k * 2 + 4 * k + 8
    return {"workload": "bf16 output layer 262144x1152 + first-max argmax", "us": round(ms * 1e3, 2),
            "GB/s": round(nbytes / ms / 1e6, 1), "frac_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
            "idx": int(idx.item())}


def bench_sketch(dev, stream, reps=50, copies=6, tokens=32):
    """The sketch head on the output layer: time per token with the tables
    rotated over `copies` weight/sketch pairs (so they come from HBM, not the
    256 MB last-level cache), the same on one pair (cache-resident), and how
    often it picks the exact argmax: on random hidden states, and on peaked
    ones (x close to one word's row, like a confident model)."""
    import numpy as np
    import torch
    from ternary_matvec_amd import qmv, synth
    v, k = synth.HEAD_V, synth.HEAD_K
    w0 = synth.normal_torch(synth.stream_seed(3, 0, 0, synth.TAG_HEAD), (v, k), std=0.02, device=dev)
    ws_ = [w0.to(torch.bfloat16)]
    del w0
    for _ in range(copies - 1):
        ws_.append(ws_[0].clone())
    sk = [qmv.qmv_sketch_build(w) for w in ws_]
    torch.cuda.synchronize()
    wsp = qmv._alloc_aligned(qmv.qmv_sketch_workspace_bytes(v, k), dev)
    xs = [torch.from_numpy(synth.normal(synth.stream_seed(3, 1, t, synth.TAG_ACT), (k,))).to(dev)
          for t in range(tokens)]
    idx = torch.empty(1, dtype=torch.int32, device=dev)
    mx = torch.empty(1, dtype=torch.float32, device=dev)
    nc = torch.empty(1, dtype=torch.int32, device=dev)

    def timed(n_pairs):
        for i in range(5):
            qmv.qmv_lmhead_sketch_argmax(ws_[i % n_pairs], sk[i % n_pairs], xs[i % tokens], idx=idx, max_logit=mx,
                                         candidates=nc, workspace=wsp, stream=stream)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(reps):
            qmv.qmv_lmhead_sketch_argmax(ws_[i % n_pairs], sk[i % n_pairs], xs[i % tokens], idx=idx, max_logit=mx,
                                         candidates=nc, workspace=wsp, stream=stream)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    ms_hbm = timed(copies)
    ms_cached = timed(1)
    # agreement with the exact search, and the candidate counts
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
                x = (8.0 * wf[r] + torch.from_numpy(synth.normal(synth.stream_seed(3, 2, t, synth.TAG_ACT),
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
            "us": round(ms_hbm * 1e3, 2), "us_cache_resident": round(ms_cached * 1e3, 2),
            "weight_copies": copies, "bytes_per_token": int(nbytes), "GB/s": round(nbytes / ms_hbm / 1e6, 1),
            "candidates_mean": round(cand, 1),
            "agrees_with_exact_argmax": {k_: "%d/%d" % (a, tokens) for k_, a in agree.items()}}


def bench_ffn_chain(stack, dev, stream, tokens=50):
    """The feed-forward half of every layer as a dependent chain per token:
    RMSNorm -> int8 (qmv_rmsnorm_quantize), gate and up (one grouped qmv_gemv),
    GeLU(gate) * up -> int8 (qmv_glu_quantize), down (qmv_gemv): 4 launches a
    layer, 104 a token, on copy 0 of the decode stack's Gemma weights.  Also the
    fused steps alone."""
    import ctypes
    import torch
    from ternary_matvec_amd import qmv, synth
    mats = [name for (name, _, _) in stack.mats]
    gi, ui, di = mats.index("gate"), mats.index("up"), mats.index("down")
    nm = len(mats)
    hidden = stack.mats[gi][2]
    inter = stack.mats[gi][1]
    h = torch.from_numpy(synth.normal(synth.stream_seed(7, 0, 0, synth.TAG_ACT), (1, hidden))).to(dev)
    gamma = torch.from_numpy(synth.normal(synth.stream_seed(7, 1, 0, synth.TAG_ACT), (hidden,)) * 0.1 + 1.0).to(dev)
    x8a = torch.empty((1, hidden), dtype=torch.int8, device=dev)
    sxa = torch.empty(1, dtype=torch.float32, device=dev)
    yg = torch.empty((1, inter), dtype=torch.float32, device=dev)
    yu = torch.empty((1, inter), dtype=torch.float32, device=dev)
    x8b = torch.empty((1, inter), dtype=torch.int8, device=dev)
    sxb = torch.empty(1, dtype=torch.float32, device=dev)
    yd = torch.empty((1, hidden), dtype=torch.float32, device=dev)

    def prob(i, x8, sx, y):
        p = qmv.qmv_problem()
        p.w = stack.arrays[0][i].w
        p.x8, p.sx, p.m, p.y, p.acc = x8.data_ptr(), sx.data_ptr(), 1, y.data_ptr(), None
        return p

    layers = []
    for layer in range(stack.layers):
        gu = (qmv.qmv_problem * 2)(prob(layer * nm + gi, x8a, sxa, yg), prob(layer * nm + ui, x8a, sxa, yu))
        dn = (qmv.qmv_problem * 1)(prob(layer * nm + di, x8b, sxb, yd))
        layers.append((qmv.gemv_plan(gu, stream=stream), qmv.gemv_plan(dn, stream=stream)))
    torch.cuda.synchronize()

    def token():
        for gu, dn in layers:
            qmv.qmv_rmsnorm_quantize(h, gamma, 1e-6, x8=x8a, sx=sxa, stream=stream)
            gu.launch(stream)
            qmv.qmv_glu_quantize(yg, yu, qmv.QMV_ACT_GELU_TANH, x8=x8b, sx=sxb, stream=stream)
            dn.launch(stream)

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(reps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps * 1e3

    us = timed(token, tokens)
    # the same 104 launches captured once in a HIP graph and replayed
    torch.cuda.synchronize()
    yd_eager = None
    token()
    torch.cuda.synchronize()
    yd_eager = yd.clone()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for gu, dn in layers:
                qmv.qmv_rmsnorm_quantize(h, gamma, 1e-6, x8=x8a, sx=sxa, stream=cap)
                gu.launch(cap)
                qmv.qmv_glu_quantize(yg, yu, qmv.QMV_ACT_GELU_TANH, x8=x8b, sx=sxb, stream=cap)
                dn.launch(cap)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    replays_match = True
    for _ in range(3):
        yd.zero_()
        graph.replay()
        torch.cuda.synchronize()
        replays_match = replays_match and bool(torch.equal(yd, yd_eager))
    us_graph = timed(graph.replay, tokens)
    wbytes = stack.layers * sum(n * ((k + 4) // 5) for (name, n, k) in stack.mats if name in ("gate", "up", "down"))
    x512 = torch.from_numpy(synth.normal(synth.stream_seed(7, 2, 0, synth.TAG_ACT), (512, hidden))).to(dev)
    g512 = torch.from_numpy(synth.normal(synth.stream_seed(7, 3, 0, synth.TAG_ACT), (512, inter))).to(dev)
    u512 = torch.from_numpy(synth.normal(synth.stream_seed(7, 4, 0, synth.TAG_ACT), (512, inter))).to(dev)
    r1 = timed(lambda: qmv.qmv_rmsnorm_quantize(h, gamma, 1e-6, x8=x8a, sx=sxa, stream=stream), 200)
    r512 = timed(lambda: qmv.qmv_rmsnorm_quantize(x512, gamma, 1e-6, stream=stream), 50)
    g1 = timed(lambda: qmv.qmv_glu_quantize(yg, yu, qmv.QMV_ACT_GELU_TANH, x8=x8b, sx=sxb, stream=stream), 200)
    g5 = timed(lambda: qmv.qmv_glu_quantize(g512, u512, qmv.QMV_ACT_GELU_TANH, stream=stream), 50)
    return {"workload": "Gemma-3-1B FFN half x26 layers, batch 1, dependent: rmsnorm->int8, gate+up GEMV, "
                        "GeLU(gate)*up->int8, down GEMV (104 launches a token)",
            "us_per_token": round(us, 1), "us_per_token_graph_replay": round(us_graph, 1),
            "graph_replays_match_eager": replays_match,
            "weight_bytes": wbytes, "GB/s": round(wbytes / us / 1e3, 1),
            "rmsnorm_quantize_us": {"1x%d" % hidden: round(r1, 2), "512x%d" % hidden: round(r512, 2)},
            "glu_quantize_us": {"1x%d" % inter: round(g1, 2), "512x%d" % inter: round(g5, 2)}}


def bench_int8(dev, stream, reps=2000):
    import torch
    from ternary_matvec_amd import qmv, synth
    n, k = synth.INT8_N, synth.INT8_K
    w = torch.from_numpy(synth.normal(synth.stream_seed(0, 0, 0, synth.TAG_WEIGHT), (n, k), std=0.02)).to(dev)
    x = torch.from_numpy(synth.normal(synth.stream_seed(0, 0, 0, synth.TAG_ACT), (1, k))).to(dev)
    pw = qmv.qmv_pack_int8(w)
    x8, sx = qmv.qmv_quantize_act(x)
    p = qmv.Problem(pw, x8, sx)
    arr = qmv.problem_array([p])
    plan = qmv.gemv_plan(arr)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        qmv.qmv_quantize_act(x, x8=x8, sx=sx, stream=stream)
        plan.launch(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / reps * 1e3
    nbytes = n * k + 5 * k + 4 * n + 8
    return {"workload": "int8 per-tensor GEMV 768x288, batch 1 (quantise + GEMV)", "us_per_call": round(us, 2),
            "GB/s": round(nbytes / us / 1e3, 2)}


def bench_groupscale(dev, stream, copies=2, reps=50):
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
    arrays, plans = [], []
    for c in range(copies):
        probs = []
        for i, (n, k, o, nb, so, ns) in enumerate(descs):
            wc = qmv.Weight(qmv.qmv_weight(qmv.QMV_W_INT8_G128, 0, n, k, pools[c][o:].data_ptr(),
                                           spool[c][so:].data_ptr()), pools[c][o:o + nb], spool[c][so:so + ns])
            probs.append(qmv.Problem(wc, acts[i][0], acts[i][1], y=ys[i]))
        arr = qmv.problem_array(probs)
        arrays.append(arr)
        plans.append(qmv.gemv_plan(arr))
    torch.cuda.synchronize()
    for i in range(10):
        plans[i % copies].launch(stream)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(reps):
        plans[i % copies].launch(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / reps * 1e3
    nbytes = wbytes + 4 * nscale + sum(k + 4 * ((k + 31) // 32) + 4 * n for (_, _, n, k) in specs)
    out = {"workload": "int8 weights in groups of 128 columns, activation scales per 32, Gemma-3-1B shapes x26 "
                       "(156 matrices), batch 1, one grouped launch", "weight_copies": copies,
           "bytes_per_launch": nbytes, "us_per_launch": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
           "frac_of_8TBps": round(nbytes / us / 8e6, 3)}
    del pools, spool, arrays, plans
    torch.cuda.empty_cache()
    return out


def bench_bitnet(dev, stream, steps, warmup, copies):
    import torch
    from ternary_matvec_amd import synth
    out = {}
    for m in (1, 4, 16):
        st = DecodeStack(synth.BITNET_MATS, synth.BITNET_LAYERS, synth.CONFIG_BITNET, m, copies, dev)
        step_ms, gemv_ms, _ = time_decode(st, steps, warmup, stream)
        out["m%d" % m] = {"gemv_us": round(gemv_ms * 1e3, 2), "step_us": round(step_ms * 1e3, 2),
                          "gemv_GB/s": round(st.gemv_bytes() / gemv_ms / 1e6, 1),
                          "weights_per_s": float("%.4g" % (sum(n * k for (_, _, _, n, k, _) in st.specs) / gemv_ms * 1e3)),
                          "MAC/s": float("%.4g" % (st.macs() / gemv_ms * 1e3))}
        del st
        torch.cuda.empty_cache()
    return out


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
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over the dispatches of the headline launch),
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


def main():
    args = parse()
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

    log("building the Gemma-shaped decode stack (26 layers x 6 matrices, %d copies)" % args.copies)
    t0 = time.perf_counter()
    stack = DecodeStack(synth.GEMMA_MATS, synth.GEMMA_LAYERS, synth.CONFIG_GEMMA_DECODE, 1, args.copies, dev)
    log("stack ready in %.1f s: %.1f MB packed per copy" % (time.perf_counter() - t0, stack.packed_bytes / 1e6))

    step_ms, gemv_ms, wall = time_decode(stack, args.steps, args.warmup, stream)
    gemv_only_ms = time_gemv_only(stack, args.steps, args.warmup, stream)
    log("step %.2f us, gemv (events in step) %.2f us, gemv back-to-back %.2f us" %
        (step_ms * 1e3, gemv_ms * 1e3, gemv_only_ms * 1e3))

    ceiling_gbs, ceiling_ms = time_read_ceiling(stack, 50, stream)
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
                   "step": "qmv_quantize_act_many (both widths, one launch) + one grouped qmv_gemv",
                   "step_bytes": step_bytes, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "k_gemv_stream<1,1> (grouped ternary GEMV)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": gemv_traffic(),
                     "bytes_per_launch": gemv_bytes, "launch_us": round(gemv_ms * 1e3, 3),
                     "launch_us_back_to_back": round(gemv_only_ms * 1e3, 3),
                     "measured_read_ceiling": round(ceiling_gbs, 1),
                     "frac_of_measured_ceiling": round(achieved / ceiling_gbs, 4),
                     "ceiling_kernel": "qmv_read_probe: one non-temporal 16-byte-load read of the same weight copies "
                                       "(%.1f MB in %.2f us)" % (stack.pool[0].numel() / 1e6, ceiling_ms * 1e3)},
    }
    log("prefill (512 tokens)")
    result["prefill"] = bench_prefill(stack, dev, stream, per_matrix=not (args.no_extras or args.profile_set))
    log("prefill %.1f us, %.1f TOPS" % (result["prefill"]["prefill_us"], result["prefill"]["TOPS"]))
    if args.profile_set and not args.no_extras:
        log("output layer")
        result["extras"] = {"lmhead": bench_head(dev, stream)}
        torch.cuda.empty_cache()
        log("sketch head")
        result["extras"]["lmhead_sketch"] = bench_sketch(dev, stream)
        torch.cuda.empty_cache()
        log("group-scaled int8 decode")
        result["extras"]["groupscale_decode"] = bench_groupscale(dev, stream)
    elif not args.no_extras:
        extras = {}
        try:
            log("decode variants")
            extras["decode_copies_sweep"] = copies_sweep(stack, max(20, args.steps // 2), stream)
            extras["decode_chained"] = chained(stack, max(5, args.steps // 20), stream)
            extras["quantize_step"] = time_quantize(stack, max(20, args.steps // 2), stream)
            log("FFN chain")
            extras["ffn_chain"] = bench_ffn_chain(stack, dev, stream)
            log("output layer")
            extras["lmhead"] = bench_head(dev, stream)
            torch.cuda.empty_cache()
            log("sketch head")
            extras["lmhead_sketch"] = bench_sketch(dev, stream)
            extras["lmhead_sketch"]["speedup_vs_full_head"] = round(extras["lmhead"]["us"] /
                                                                    extras["lmhead_sketch"]["us"], 2)
            torch.cuda.empty_cache()
            log("int8 GEMV")
            extras["int8_gemv"] = bench_int8(dev, stream)
            log("group-scaled int8 decode")
            extras["groupscale_decode"] = bench_groupscale(dev, stream)
            log("BitNet decode")
            extras["bitnet_decode"] = bench_bitnet(dev, stream, max(20, args.steps // 4), 5, min(args.copies, 8))
        except Exception as e:  # extras never hide the headline line
            extras["error"] = repr(e)
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
        result["cpu_baseline"] = cpu_baseline(stack, args.cpu_seconds, dev)
        if not args.no_extras:
            result.setdefault("extras", {})["cpu_oracle_1_thread"] = cpu_single_thread(stack, 3.0, dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
