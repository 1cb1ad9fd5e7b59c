"""Pins for unused parameters in the oracle ([Li] "Handling Unused Parameters
and Sub-Graph Execution", [TP] forward pass and "When a parameter never
receives a gradient", [C30] "Unused Parameter"): globally unused variables are
treated as ready and their gradients left alone; a replica that did not use a
variable contributes zeros; the used flags are OR-ed over replicas and over
no_sync micro-steps."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import reducer as OR
from workloads import gen as WG
from test_oracle_reducer import round_to_f32


def _red(numels, R, cap, seed=0, view=False):
    red = OR.Reducer(numels, R, cap, gradient_as_bucket_view=view)
    grads = [[WG.dyadic(seed * 1000 + 37 * r + v, n) for v, n in enumerate(numels)] for r in range(R)]
    if view:
        for r in range(R):
            for v in range(len(numels)):
                red.views()[r][v][...] = grads[r][v]
        return red, red.views(), [[g.copy() for g in row] for row in grads]
    local = [[g.copy() for g in row] for row in grads]
    red.bind(grads)
    return red, grads, local


def test_skipped_without_marking_fails_and_marking_completes():
    numels = [4, 4, 4]
    red, _, _ = _red(numels, 2, 0)
    red.mark_ready(2)
    red.mark_ready(1)
    with pytest.raises(OR.ReductionIncomplete):
        red.finalize()
    red2, grads, local = _red(numels, 2, 0)
    red2.set_local_used([[False, True, True], [False, True, True]])   # no replica uses variable 0
    red2.sync([2, 1])
    # globally unused variable 0: gradients untouched on every replica
    for r in range(2):
        assert np.array_equal(grads[r][0], local[r][0])
    assert [b for b, _ in red2.launch_log] == [0, 1, 2]


@pytest.mark.parametrize("R", [2, 3, 5, 8])
def test_locally_unused_replicas_contribute_zeros(R):
    numels = [6, 9, 3]
    red, grads, local = _red(numels, R, 4 * 10, seed=R)
    red.sync()                                 # an earlier iteration leaves data in every slice
    for r in range(R):
        for v in range(3):
            grads[r][v][...] = local[r][v]
    rng = np.random.default_rng(R)
    used = rng.random((R, 3)) < 0.6
    used[0, :] = True                          # every variable used somewhere
    red.set_local_used(used)
    red.sync()
    for v, n in enumerate(numels):
        for i in range(n):
            exact = sum(Fraction(float(local[r][v][i])) for r in range(R) if used[r, v]) / R
            want = round_to_f32(exact)
            for r in range(R):                 # the global mean reaches every replica
                assert grads[r][v][i].view(np.uint32) == want.view(np.uint32), (v, i, r)


def test_marking_an_unused_variable_twice_is_an_error():
    red, _, _ = _red([4, 4], 2, 0)
    red.set_local_used([[True, False], [True, False]])
    red.mark_ready(0)                          # first hook marks variable 1 ready as unused
    with pytest.raises(OR.DoubleReady):
        red.mark_ready(1)


def test_used_flags_accumulate_over_no_sync_steps():
    numels = [5, 7]
    R, k = 2, 3
    red = OR.Reducer(numels, R, 0)
    g = [[np.zeros(n, np.float32) for n in numels] for _ in range(R)]
    red.bind(g)
    steps = [[[WG.dyadic(100 * t + 10 * r + v, n) if (v == 0 or t == 1) else None
               for v, n in enumerate(numels)] for r in range(R)] for t in range(k)]
    red.set_sync(False)
    for t in range(k):
        if t == k - 1:
            red.set_sync(True)
        red.set_local_used([[True, t == 1]] * R)   # variable 1 only used in micro-step 1
        red.no_sync_accumulate(steps[t], first=(t == 0))
        red.sync()
    assert red.used_acc is None                # consumed by the synchronisation
    # variable 1 counts as used: its gradient (step 1 only) is averaged
    want = OR.fixed_order_mean([steps[1][r][1] for r in range(R)])
    for r in range(R):
        assert np.array_equal(g[r][1], want)


def test_all_variables_unused_still_finishes():
    red, grads, local = _red([4, 4], 2, 0)
    red.set_local_used(np.zeros((2, 2), bool))
    red.finalize()                             # no hook fires at all
    assert [b for b, _ in red.launch_log] == [0, 1]
    for r in range(2):
        for v in range(2):
            assert np.array_equal(grads[r][v], local[r][v])


def test_bucket_view_mode_zero_fills_unused_views():
    numels = [4, 6, 3]
    R = 3
    red, views, local = _red(numels, R, 0, view=True)
    used = np.array([[True, False, True], [True, False, False], [True, False, True]])
    red.set_local_used(used)
    red.sync([2, 0])
    assert np.all(views[0][1] == 0) and np.all(views[2][1] == 0)   # globally unused: the zeroed slice
    want = OR.fixed_order_mean([local[0][2], np.zeros(3, np.float32), local[2][2]])
    for r in range(R):
        assert np.array_equal(views[r][2], want)


def test_rebuild_is_refused_after_an_iteration_with_unused_variables():
    red, _, _ = _red([4, 4, 4], 2, 0)
    red.set_local_used([[True, False, True]] * 2)
    red.sync([2, 0])
    assert red.rebuild_buckets() is False


def test_planted_unused_mistakes_are_caught(monkeypatch):
    # (a) stale gradients of replicas that did not use a variable
    real = OR.Reducer._zero_slices
    monkeypatch.setattr(OR.Reducer, "_zero_slices", lambda self, r, v: None)
    with pytest.raises(AssertionError):
        test_locally_unused_replicas_contribute_zeros(3)
    monkeypatch.setattr(OR.Reducer, "_zero_slices", real)
    # (b) AND instead of OR over no_sync steps
    def and_used(self, used):
        u = np.asarray(used, dtype=bool).reshape(self.R, self.P)
        self.used_acc = u.copy() if self.used_acc is None else (self.used_acc & u)
    monkeypatch.setattr(OR.Reducer, "set_local_used", and_used)
    with pytest.raises((AssertionError, OR.DoubleReady)):
        test_used_flags_accumulate_over_no_sync_steps()


def _first_hook_names_an_unused_variable(cls):
    """The iteration's first hook names a variable already marked ready as
    unused (DoubleReady); the remaining hooks must still complete it, with the
    unused marking applied once: cap 0, v2 -> bucket 0, v1 -> 1, v0 -> 2."""
    red = cls([4, 4, 4], 2, 0)
    g = [[WG.dyadic(50 + 3 * r + v, 4) for v in range(3)] for r in range(2)]
    local = [[x.copy() for x in row] for row in g]
    red.bind(g)
    red.set_local_used([[True, False, True], [True, False, True]])
    with pytest.raises(OR.DoubleReady):
        red.mark_ready(1)
    red.mark_ready(2)
    red.mark_ready(0)
    red.finalize()
    assert red.launch_log == [(0, 0), (1, 0), (2, 1)]
    for r in range(2):
        assert np.array_equal(g[r][1], local[r][1])                  # unused: untouched
        assert np.array_equal(g[r][0], OR.fixed_order_mean([local[0][0], local[1][0]]))


def test_unused_marking_happens_once_even_after_a_failed_first_hook():
    _first_hook_names_an_unused_variable(OR.Reducer)


def test_planted_repeated_unused_marking_is_caught():
    class Remarks(OR.Reducer):                   # keys the marking on the call count instead
        def mark_ready(self, v):
            if self.calls == 0:
                self.started = False
            return super().mark_ready(v)
    with pytest.raises((AssertionError, OR.ReductionIncomplete)):
        _first_hook_names_an_unused_variable(Remarks)
