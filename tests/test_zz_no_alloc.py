"""qmv_lmhead_argmax_static (no workspace, nothing allocated) against
qmv_lmhead_argmax on the same inputs, through the C ABI: two calls in a row on
one device, the second with a smaller table, so the shared scratch array holds
the first call's maxima when the second starts.  The two entry points run the
same kernels, so the index, the maximum and every logit must be identical."""
import sys

import numpy as np
import pytest
import torch

from ternary_matvec_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _inputs(v, k, seed):
    w = synth.to_bf16_bits(synth.normal(seed, (v, k), std=0.02))
    x = synth.normal(seed + 1, (k,))
    return torch.from_numpy(w.view(np.int16)).to(DEV), torch.from_numpy(x).to(DEV)


def test_static_entry_point_matches_workspace_entry_point(qmv_gpu):
    from ternary_matvec_amd import qmv
    for v, k, seed in ((262144, 1152, 501), (3000, 96, 502)):   # second call smaller
        say("lmhead static %d x %d" % (v, k))
        w, x = _inputs(v, k, seed)
        i_s, m_s, l_s = qmv.qmv_lmhead_argmax_static(w, x, want_logits=True)
        torch.cuda.synchronize()
        i_w, m_w, l_w = qmv.qmv_lmhead_argmax(w, x, want_logits=True)
        torch.cuda.synchronize()
        assert int(i_s.item()) == int(i_w.item())
        assert m_s.cpu().numpy().view(np.uint32)[0] == m_w.cpu().numpy().view(np.uint32)[0]
        assert torch.equal(l_s.view(torch.int32), l_w.view(torch.int32))
        assert 0 <= int(i_s.item()) < v
        del w, x, l_s, l_w
        torch.cuda.empty_cache()


def test_static_entry_point_planted_winner_after_larger_call(qmv_gpu):
    from ternary_matvec_amd import qmv
    say("lmhead static planted winner in a small table after a large one")
    w, x = _inputs(100000, 256, 503)
    qmv.qmv_lmhead_argmax_static(w, x)
    torch.cuda.synchronize()
    v, k = 700, 256
    wb = synth.to_bf16_bits(synth.normal(504, (v, k), std=0.02))
    xs = synth.normal(505, (k,))
    wb[321] = synth.to_bf16_bits(np.sign(xs) * 0.5)
    idx, _, _ = qmv.qmv_lmhead_argmax_static(torch.from_numpy(wb.view(np.int16)).to(DEV),
                                             torch.from_numpy(xs).to(DEV))
    torch.cuda.synchronize()
    assert int(idx.item()) == 321
