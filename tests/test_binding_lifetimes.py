"""A struct array made by the binding keeps alive what its pointers name.

A plan uploads the device pointers of its problems once and writes the outputs
on every launch.  If the Python objects owning those tensors could be dropped
while the plan lives, the caching allocator would hand their memory to the next
allocation (the plan's own workspace, say), and later launches would write into
it.  problem_array therefore holds references to the problems it was built
from; a plan holds its array.  CPU only (the problems here are stand-ins with
the binding's struct() protocol).
"""
import gc
import weakref

from ternary_matvec_amd import qmv


class _Stand:
    def struct(self):
        return qmv.qmv_problem()


def test_problem_array_keeps_its_problems_alive():
    p = _Stand()
    ref = weakref.ref(p)
    arr = qmv.problem_array([p])
    del p
    gc.collect()
    assert ref() is not None, "the array must keep the problem (and its tensors) alive"
    del arr
    gc.collect()
    assert ref() is None


def test_problem_array_keeps_a_temporary_list_alive():
    refs = []

    def build():
        ps = [_Stand(), _Stand()]
        refs.extend(weakref.ref(p) for p in ps)
        return qmv.problem_array(ps)   # the list and its problems go out of scope here

    arr = build()
    gc.collect()
    assert all(r() is not None for r in refs)
    assert len(arr) == 2
