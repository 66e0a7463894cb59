"""Host-side behaviour of bench.py that needs no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""            # no JSON line for an unmeasured configuration


def test_bench_byte_accounting_matches_the_workload_definition():
    # DecodeStack's accounting methods applied to the headline shapes without a
    # GPU: packed weights N * ceil(K/5), int8 activations K, fp32 outputs 4N and
    # the two scales per matrix; the quantiser reads 4 B and writes 1 B per
    # activation plus a 4-byte scale per row
    sys.path.insert(0, ROOT)
    import numpy as np
    import bench
    from ternary_matvec_amd import synth

    class Shape:
        def __init__(self, rows, k):
            self.shape = (rows, k)

        def numel(self):
            return self.shape[0] * self.shape[1]

    st = bench.DecodeStack.__new__(bench.DecodeStack)
    st.m = 1
    st.specs = [(layer, mid, name, n, k, 0) for layer in range(synth.GEMMA_LAYERS)
                for mid, (name, n, k) in enumerate(synth.GEMMA_MATS)]
    st.x = {1152: Shape(130, 1152), 6912: Shape(26, 6912)}
    assert st.weight_bytes() == 133675776
    assert st.gemv_bytes() == 135723744
    assert st.quant_bytes() == 5 * (130 * 1152 + 26 * 6912) + 4 * 156
    assert st.step_bytes() == st.gemv_bytes() + st.quant_bytes()
    assert np.isclose(st.step_bytes(), 137371728)
