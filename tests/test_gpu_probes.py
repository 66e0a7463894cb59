"""The measurement aids run to completion and leave the result word alone
unless the folded value hits the key: the plain read over a buffer of known
contents (the word is written only when the xor of everything read equals
the key), and the register-only matrix-instruction stream, whose operation
count follows from the launch shape."""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KEY = 0x9e3779b9


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def test_read_probe_reads_everything(qmv_gpu):
    from ternary_matvec_amd import qmv
    say("read probe")
    # 64 MiB of ones: every lane's xor of an even number of all-ones words is 0
    buf = torch.full((64 << 20,), 0xFF, dtype=torch.uint8, device=DEV)
    out = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    qmv.qmv_read_probe(buf, out)
    torch.cuda.synchronize()
    assert int(out.item()) == 7
    # a buffer whose words xor to the key from one lane: the word is written
    small = torch.zeros(16, dtype=torch.uint8, device=DEV)
    small.view(torch.int32)[0] = KEY - (1 << 32)
    qmv.qmv_read_probe(small, out)
    torch.cuda.synchronize()
    assert int(out.item()) & 0xFFFFFFFF == KEY


@pytest.mark.parametrize("kind", [0, 1])
def test_mfma_probe_runs(qmv_gpu, kind):
    from ternary_matvec_amd import qmv
    say("matrix probe", kind)
    out = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    iters = 64
    ops = qmv.qmv_mfma_probe(kind, iters, out)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    chains, per = (6, 2 * 16 * 16 * 64) if kind == 0 else (8, 2 * 32 * 32 * 32)
    assert ops == cus * 4 * 4 * iters * chains * per
    assert int(out.item()) in (7, KEY - (1 << 32))
