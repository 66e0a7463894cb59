"""The int8 matrix instructions in the built kernels keep their accumulators in
place: the assembly hipcc emits for gfx950 (from these sources, with the
library's flags) has, for every v_mfma, result registers that are either the
accumulator-input registers themselves or disjoint from them.  A partial
overlap (e.g. result a[24:27] from accumulator a[22:25]) is an operand layout
these kernels never rely on; hipcc can emit one when accumulators start from
constants, so a change that did so would fail here.  CPU only: cross-compiles.
"""
import os
import re
import subprocess
import tempfile

import pytest

from ternary_matvec_amd import build

MFMA_SOURCES = ("k_gemv_mx.hip", "k_prefill.hip", "k_probe.hip")
REG = re.compile(r"^([av])\[(\d+):(\d+)\]$|^([av])(\d+)$")


def _range(tok):
    m = REG.match(tok)
    assert m, tok
    if m.group(1):
        return m.group(1), int(m.group(2)), int(m.group(3))
    return m.group(4), int(m.group(5)), int(m.group(5))


def _mfma_operands(asm):
    for line in asm.splitlines():
        line = line.strip()
        if not line.startswith("v_mfma"):
            continue
        ops = [t.strip() for t in line.split(None, 1)[1].split(",")]
        yield line, _range(ops[0]), _range(ops[3].split()[0])


def _overlap_ok(d, c):
    if d[0] != c[0]:
        return True
    if (d[1], d[2]) == (c[1], c[2]):
        return True
    return d[2] < c[1] or c[2] < d[1]


def test_overlap_rule_itself():
    assert _overlap_ok(("a", 0, 3), ("a", 0, 3))
    assert _overlap_ok(("a", 4, 7), ("a", 0, 3))
    assert _overlap_ok(("v", 0, 3), ("a", 0, 3))
    assert not _overlap_ok(("a", 24, 27), ("a", 22, 25))
    assert not _overlap_ok(("a", 12, 15), ("a", 10, 13))


@pytest.mark.parametrize("src", MFMA_SOURCES)
def test_mfma_accumulators_never_partially_overlap(src):
    path = os.path.join(build.CSRC, src)
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [build.HIPCC] + [f for f in build.CFLAGS if f != "-fPIC"] + ["-S", "--cuda-device-only", path,
                                                                           "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        asm = open(out).read()
    seen = 0
    for line, dst, acc in _mfma_operands(asm):
        seen += 1
        assert _overlap_ok(dst, acc), line
    assert seen > 0
