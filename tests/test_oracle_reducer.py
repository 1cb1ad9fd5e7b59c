"""Pins for the oracle's readiness state machine, fixed-order mean, copy-back,
finalize and no_sync accumulation."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from conftest import load_golden
from oracle import reducer as OR
from workloads import gen as WG

MiB = 1 << 20


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def round_to_f32(q: Fraction) -> np.float32:
    """Round a rational to the nearest binary32 value, ties to even, with
    subnormals (straight from the definition of IEEE-754 rounding)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                     # now 2^e <= a < 2^(e+1)
    ulp = Fraction(2) ** (max(e, -126) - 23)
    n = a / ulp
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    val = k * ulp
    assert val < Fraction(2) ** 128
    return np.float32(sign * float(val))           # exact: val is a binary32 value


def _make(numels, R, cap, seed=0, dyadic=False):
    red = OR.Reducer(numels, R, cap)
    if dyadic:
        grads = [[WG.dyadic(seed * 1000 + r * 100 + v, n) for v, n in enumerate(numels)] for r in range(R)]
    else:
        rng = np.random.default_rng(seed)
        grads = [[(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in numels] for r in range(R)]
    local = [[g.copy() for g in row] for row in grads]
    red.bind(grads)
    return red, grads, local


# --- launch order --------------------------------------------------------------

def test_printed_in_order_sequence():
    g = load_golden("c30_inorder_sequence.json")
    # three one-tensor buckets: bucket b holds variable 2 - b
    red, _, _ = _make([4, 4, 4], 2, 0)
    assert red.buckets == [[2], [1], [0]]
    for ev in g["events"]:
        before = len(red.launch_log)
        red.mark_ready(red.buckets[ev["bucket_completes"]][0])
        assert [b for b, _ in red.launch_log[before:]] == ev["launched_after"]
    red.finalize()


def _closed_form_launch_calls(buckets, order):
    # c_b = the call at which bucket b's last member is marked; bucket b is
    # launched at call max_{b' <= b} c_{b'}
    pos = {v: i for i, v in enumerate(order)}
    c = [max(pos[v] for v in b) for b in buckets]
    return [(b, max(c[:b + 1])) for b in range(len(buckets))]


def test_launch_order_closed_form_all_permutations():
    rng = np.random.default_rng(3)
    checked = 0
    for P in range(1, 7):
        for trial in range(3):
            numels = [int(x) for x in rng.integers(1, 9, size=P)]
            cap = int(rng.integers(0, 4 * sum(numels) // 2 + 1))
            for order in itertools.permutations(range(P)):
                red, _, _ = _make(numels, 2, cap, seed=trial)
                red.sync(order)
                assert red.launch_log == _closed_form_launch_calls(red.buckets, order)
                checked += 1
    assert checked > 1000


def test_launch_order_closed_form_random_large():
    for seed in range(20):
        P = 60
        numels = WG.random_numels(seed, P, 1, 50)
        red, _, _ = _make(numels, 3, 200, seed=seed)
        order = WG.permutation(seed, P)
        red.sync(order)
        assert red.launch_log == _closed_form_launch_calls(red.buckets, order)
        assert [b for b, _ in red.launch_log] == list(range(red.B))


def test_reverse_index_ready_order_matches_printed_hook_order():
    g = load_golden("c30_ready_order.json")
    red, _, _ = _make([MiB] * g["params"], 1, 4 * MiB)
    assert list(reversed(range(g["params"]))) == g["ready_order"]
    red.sync(g["ready_order"])
    # each 4 MiB tensor is its own bucket and is launched by its own hook
    assert red.launch_log == [(b, b) for b in range(12)]


# --- results -------------------------------------------------------------------

def test_different_ready_orders_give_identical_results():
    g = load_golden("li_fig3a_orders.json")
    numels = [7, 5, 9, 3]
    outs, contents = [], []
    for order1 in g["process_orders_1based"]:
        order = [i - 1 for i in order1]
        red, grads, _ = _make(numels, 4, 40, seed=11)
        assert red.B == 2
        red.sync(order)
        outs.append([[_bits(x).copy() for x in row] for row in grads])
        contents.append([[_bits(b).copy() for b in row] for row in red.flat])
    for a, b in zip(outs[0], outs[1]):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    for a, b in zip(contents[0], contents[1]):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("R", [1, 2, 3, 5, 7, 8, 16])
def test_every_replica_gets_exact_rounded_mean_on_dyadic_inputs(R):
    # integers in [-2^10, 2^10] times 2^-12: every partial sum of <= 16 terms
    # is exact in float32, so the only rounding is the final division.
    numels = [37, 1, 130, 64]
    red, grads, local = _make(numels, R, 300, seed=R, dyadic=True)
    red.sync()
    for v, n in enumerate(numels):
        for i in range(n):
            exact = sum(Fraction(float(local[r][v][i])) for r in range(R)) / R
            want = round_to_f32(exact)               # one rounding of the exact mean
            for r in range(R):
                assert _bits(grads[r][v][i]) == _bits(want), (R, v, i)


def test_mean_error_bound_general_inputs():
    rng = np.random.default_rng(5)
    for R in (2, 3, 8, 16):
        bufs = [rng.standard_normal(4096).astype(np.float32) * np.float32(10.0 ** rng.integers(-3, 3))
                for _ in range(R)]
        m = OR.fixed_order_mean(bufs).astype(np.float64)
        exact = np.sum([b.astype(np.float64) for b in bufs], axis=0) / R
        u = 2.0 ** -24
        gamma = (R - 1) * u / (1 - (R - 1) * u)
        bound = gamma * np.sum([np.abs(b.astype(np.float64)) for b in bufs], axis=0) / R + u * np.abs(exact)
        assert np.all(np.abs(m - exact) <= bound * (1 + 1e-12) + 1e-45)


def test_mean_special_cases():
    x = np.array([1.5, -2.25, 3e-39, np.float32(1) / np.float32(3)], dtype=np.float32)
    assert np.array_equal(_bits(OR.fixed_order_mean([x])), _bits(x))          # R = 1: identity
    assert np.array_equal(_bits(OR.fixed_order_mean([x, x])), _bits(x))       # R = 2, equal replicas
    # left-to-right order from rank 0: fl(2^24 + 1) = 2^24, minus 2^24 = 0
    a = [np.array([2.0 ** 24], np.float32), np.array([1.0], np.float32), np.array([-(2.0 ** 24)], np.float32)]
    assert OR.fixed_order_mean(a)[0] == 0.0
    # subnormals are kept, not flushed: (2^-149 + 2^-149) / 2 = 2^-149
    tiny = np.array([np.float32(2.0 ** -149)], np.float32)
    assert _bits(OR.fixed_order_mean([tiny, tiny]))[0] == 1
    # true division: mean of {1, 0, 0} is the float nearest to 1/3
    t = OR.fixed_order_mean([np.array([1.0], np.float32), np.zeros(1, np.float32), np.zeros(1, np.float32)])
    assert t[0] == np.float32(1.0 / 3.0)


def test_hook_divides_by_world_size():
    # forgetting the division is the silent bug the pages warn about
    red, grads, local = _make([16], 4, 0, dyadic=True)
    red.sync()
    s = np.sum([local[r][0].astype(np.float64) for r in range(4)], axis=0)
    assert np.array_equal(grads[0][0].astype(np.float64), s / 4)
    assert not np.array_equal(grads[0][0].astype(np.float64), s) or np.all(s == 0)


def test_flat_bucket_views_hold_packed_gradients():
    numels = [3, 5, 2]
    red, grads, local = _make(numels, 2, 10 ** 9, seed=1)   # one bucket, order [2, 1, 0]
    for v in (2, 1):
        red.mark_ready(v)
    L = red.loc[1]
    assert np.array_equal(red.flat[1][0][L.offset:L.offset + L.length], local[1][1])
    assert red.loc[2].offset == 0 and red.loc[1].offset == 2 and red.loc[0].offset == 7
    red.mark_ready(0)
    red.finalize()


# --- errors --------------------------------------------------------------------

def test_incomplete_reduction_surfaces_at_next_iteration():
    red, _, _ = _make([4, 4, 4], 2, 0)
    red.mark_ready(2)
    red.mark_ready(1)          # variable 0 never receives a gradient
    with pytest.raises(OR.ReductionIncomplete):
        red.finalize()
    with pytest.raises(OR.ReductionIncomplete):
        red.mark_ready(2)
    with pytest.raises(OR.ReductionIncomplete):
        red.ensure_prior_reduction_finished()
    red.reset()
    red.sync()
    red.ensure_prior_reduction_finished()


def test_unfinished_iteration_detected_before_next_forward():
    red, _, _ = _make([4, 4], 2, 0)
    red.mark_ready(1)
    with pytest.raises(OR.ReductionIncomplete):
        red.ensure_prior_reduction_finished()


def test_double_ready_and_bad_index():
    red, _, _ = _make([4, 4], 2, 0)
    red.mark_ready(1)
    with pytest.raises(OR.DoubleReady):
        red.mark_ready(1)
    with pytest.raises(IndexError):
        red.mark_ready(2)


# --- no_sync ---------------------------------------------------------------------

def test_no_sync_k_steps_equals_sync_of_summed_gradients():
    numels = [33, 8, 100]
    R, k = 4, 5
    for dyadic in (True, False):
        red = OR.Reducer(numels, R, 200)
        grads = [[np.zeros(n, np.float32) for n in numels] for _ in range(R)]
        red.bind(grads)
        steps = []
        for t in range(k):
            if dyadic:
                st = [[WG.dyadic(t * 997 + r * 31 + v, n) for v, n in enumerate(numels)] for r in range(R)]
            else:
                rng = np.random.default_rng(t)
                st = [[(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in numels] for r in range(R)]
            steps.append(st)
        red.set_sync(False)
        for t in range(k - 1):
            red.no_sync_accumulate(steps[t], first=(t == 0))
            red.sync()                  # hooks run but do nothing
            assert red.launch_log == []
        red.set_sync(True)
        red.no_sync_accumulate(steps[k - 1], first=(k == 1))
        red.sync()
        for v, n in enumerate(numels):
            summed = [steps[0][r][v].copy() for r in range(R)]
            for t in range(1, k):
                summed = [summed[r] + steps[t][r][v] for r in range(R)]
            want = OR.fixed_order_mean(summed)
            for r in range(R):
                assert np.array_equal(_bits(grads[r][v]), _bits(want))
            # equals the sum over steps of per-step means: exactly on dyadic
            # inputs, within the float32 bound otherwise
            per_step = sum(OR.fixed_order_mean([steps[t][r][v] for r in range(R)]).astype(np.float64)
                           for t in range(k))
            if dyadic:
                assert np.array_equal(grads[0][v].astype(np.float64), per_step)
            else:
                assert np.allclose(grads[0][v], per_step, rtol=1e-5, atol=1e-9)


def test_no_sync_single_step_is_plain_sync():
    numels = [10, 20]
    red = OR.Reducer(numels, 2, 0)
    g1 = [[np.zeros(n, np.float32) for n in numels] for _ in range(2)]
    red.bind(g1)
    st = [[WG.dyadic(r * 10 + v, n) for v, n in enumerate(numels)] for r in range(2)]
    red.no_sync_accumulate(st, first=True)
    red.sync()
    want = [OR.fixed_order_mean([st[0][v], st[1][v]]) for v in range(2)]
    for v in range(2):
        assert np.array_equal(g1[1][v], want[v])


def test_bf16_widening_is_exact():
    vals = np.array([0.0, -0.0, 1.0, -2.5, 3.0e-3, 1e-40, np.inf], dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)      # truncation of exactly representable bf16
    back = OR.bf16_bits_to_f32(bits)
    assert np.array_equal(back.view(np.uint32), (bits.astype(np.uint32) << 16))
    assert back[2] == 1.0 and back[3] == -2.5 and np.isinf(back[6])


# --- planted mistakes --------------------------------------------------------------

def _mean_no_divide(bufs):
    acc = np.array(bufs[0], np.float32)
    for b in bufs[1:]:
        acc = acc + b
    return acc


def _mean_reverse_order(bufs):
    acc = np.array(bufs[-1], np.float32)
    for b in reversed(bufs[:-1]):
        acc = acc + b
    return acc / np.float32(len(bufs))


def _mean_drops_last(bufs):
    acc = np.array(bufs[0], np.float32)
    for b in bufs[1:-1]:
        acc = acc + b
    return acc / np.float32(len(bufs))


def _mean_reciprocal(bufs):
    acc = np.array(bufs[0], np.float32)
    for b in bufs[1:]:
        acc = acc + b
    return acc * (np.float32(1) / np.float32(len(bufs)))


@pytest.mark.parametrize("mutant", [_mean_no_divide, _mean_reverse_order, _mean_drops_last, _mean_reciprocal])
def test_planted_mean_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(OR, "fixed_order_mean", mutant)
    failures = 0
    for t in (lambda: test_every_replica_gets_exact_rounded_mean_on_dyadic_inputs(3),
              lambda: test_every_replica_gets_exact_rounded_mean_on_dyadic_inputs(8),
              test_mean_special_cases, test_hook_divides_by_world_size):
        try:
            t()
        except AssertionError:
            failures += 1
    assert failures >= 1


def test_planted_launch_order_mistake_is_caught(monkeypatch):
    # launching a bucket as soon as it is ready (no parking) must break the pins
    def eager(self, b, call):
        self._launch(b, call)
        if b == self.next_bucket:
            while self.next_bucket < self.B and self.pending[self.next_bucket] == 0:
                self.next_bucket += 1
    monkeypatch.setattr(OR.Reducer, "_mark_bucket_ready", eager)
    with pytest.raises(AssertionError):
        test_printed_in_order_sequence()


def test_planted_copyback_mistake_is_caught(monkeypatch):
    # copying back into replica 0 only must break the every-replica pin
    real = OR.Reducer._launch

    def only_rank0(self, b, call):
        m = OR.fixed_order_mean([self.flat[r][b] for r in range(self.R)])
        for v in self.buckets[b]:
            L = self.loc[v]
            self.grads[0][v][...] = m[L.offset:L.offset + L.length]
        self.launch_log.append((b, call))
    monkeypatch.setattr(OR.Reducer, "_launch", only_rank0)
    with pytest.raises(AssertionError):
        test_every_replica_gets_exact_rounded_mean_on_dyadic_inputs(3)


def test_latched_failure_refuses_finalize_until_reset():
    """[TP] "When a parameter never receives a gradient": an iteration left
    open is reported at the next forward; the reading taken here latches that
    failure, so the open iteration cannot be finalized afterwards either, and a
    reset restores normal operation."""
    red = OR.Reducer([4], 2, 0)
    g = [[np.ones(4, np.float32)], [np.ones(4, np.float32)]]
    red.bind(g)
    red.mark_ready(0)                        # every bucket launched, finalize not yet called
    with pytest.raises(OR.ReductionIncomplete):
        red.ensure_prior_reduction_finished()
    with pytest.raises(OR.ReductionIncomplete):
        red.finalize()
    red.reset()
    red.sync()
    assert len(red.launch_log) == 2
