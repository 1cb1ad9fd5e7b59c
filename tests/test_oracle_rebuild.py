"""Pins for the oracle's ready-order bucket rebuild ([C30] "第一次迭代为何不同"):
the first iteration learns the order in which gradients become ready and the
buckets are then re-packed in that order with the same cap rule."""
import itertools

import numpy as np
import pytest

from conftest import load_golden
from oracle import plan as OP
from oracle import reducer as OR
from workloads import gen as WG

MiB = 1 << 20


def _red(numels, R, cap, seed=0, view=False):
    red = OR.Reducer(numels, R, cap, gradient_as_bucket_view=view)
    if not view:
        rng = np.random.default_rng(seed)
        red.bind([[(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in numels] for _ in range(R)])
    return red


def test_printed_first_iteration_then_rebuild():
    """48 MiB of 12 x 4 MiB parameters: the first iteration runs as a single
    50,331,648-byte bucket; after the rebuild the same model forms 12, 3 or 1
    buckets at caps of 4, 16 and 64 MiB (the blog's printed layouts)."""
    single = load_golden("c30_single_bucket.json")
    table = {r["cap_bytes"]: r for r in load_golden("c30_param_granularity.json")["rows"]
             if r["name"].startswith("coarse4")}
    order = load_golden("c30_ready_order.json")["ready_order"]
    numels = [MiB] * 12
    for cap, row in table.items():
        red = _red(numels, 2, 1 << 62)
        assert [4 * x for x in red.bucket_elems] == [single["bucket_bytes"]]
        red.sync(order)
        assert red.rebuild_buckets(cap)
        assert red.B == row["buckets"]
        assert all(4 * x == row["bucket_bytes"] for x in red.bucket_elems)
        red.sync(order)


def test_rebuild_with_reverse_index_order_is_the_construction_plan():
    for seed in range(10):
        numels = WG.random_numels(seed, 30, 1, 500)
        cap = 4 * 800
        red = _red(numels, 2, cap, seed)
        before = [list(b) for b in red.buckets]
        red.sync()
        assert red.rebuild_buckets()
        assert red.buckets == before


def _launch_calls(buckets, order):
    pos = {v: i for i, v in enumerate(order)}
    c = [max(pos[v] for v in b) for b in buckets]
    return [(b, max(c[:b + 1])) for b in range(len(buckets))]


def test_rebuilt_buckets_never_wait_on_a_later_gradient():
    """After the rebuild each bucket is a run of consecutive hooks of the
    learned order, so every bucket launches at its own last hook: nothing is
    parked (checked over every order for small P, random orders beyond)."""
    rng = np.random.default_rng(1)
    cases = 0
    for P in range(1, 7):
        numels = [int(x) for x in rng.integers(1, 9, size=P)]
        cap = int(rng.integers(0, 2 * sum(numels) + 1))
        for order in itertools.permutations(range(P)):
            red = _red(numels, 2, cap)
            red.sync(order)
            red.rebuild_buckets()
            red.launch_log.clear()
            red.sync(order)
            pos = {v: i for i, v in enumerate(order)}
            own = [max(pos[v] for v in b) for b in red.buckets]
            assert red.launch_log == [(b, own[b]) for b in range(red.B)]
            assert own == sorted(own)
            cases += 1
    for seed in range(20):
        numels = WG.random_numels(seed, 80, 1, 100)
        order = WG.permutation(seed, 80)
        red = _red(numels, 3, 4 * 300, seed)
        red.sync(order)
        red.rebuild_buckets()
        red.launch_log.clear()
        red.sync(order)
        assert red.launch_log == _launch_calls(red.buckets, order)
        assert [c for _, c in red.launch_log] == sorted({max(order.index(v) for v in b) for b in red.buckets})
    assert cases == 1 + 2 + 6 + 24 + 120 + 720


def test_rebuild_packs_in_ready_order_with_the_cap_rule():
    numels = [10, 20, 30, 40, 50]
    order = [2, 0, 4, 1, 3]
    red = _red(numels, 2, 4 * 45)
    red.sync(order)
    red.rebuild_buckets()
    # 30 -> 30+10=40 -> +50=90 >= 45 closes; then 20 -> +40=60 closes
    assert red.buckets == [[2, 0, 4], [1, 3]]
    assert OP.compute_bucket_assignment_by_size(numels, 4, 4 * 45, order) == red.buckets


def test_rebuild_keeps_results_identical():
    numels = WG.random_numels(4, 40, 1, 2000)
    order = WG.permutation(4, 40)
    a = _red(numels, 4, 4 * 3000, seed=9)
    b = _red(numels, 4, 4 * 3000, seed=9)
    a.sync(order)
    a.rebuild_buckets()
    rng = np.random.default_rng(2)
    fresh = [[(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in numels] for _ in range(4)]
    for red in (a, b):
        for r in range(4):
            for v in range(40):
                red.grads[r][v][...] = fresh[r][v]
    a.sync(order)
    b.sync(order)
    for r in range(4):
        for v in range(40):
            assert np.array_equal(a.grads[r][v], b.grads[r][v])


def test_rebuild_needs_a_finished_iteration():
    red = _red([4, 4, 4], 2, 0)
    assert red.rebuild_buckets() is False          # nothing learned yet
    red.mark_ready(2)
    with pytest.raises(OR.ReductionIncomplete):
        red.rebuild_buckets()


def test_rebuild_in_bucket_view_mode_hands_out_new_views():
    numels = [7, 5, 9]
    red = _red(numels, 2, 4 * 10, view=True)
    red.sync([0, 1, 2])
    red.rebuild_buckets()
    assert red.buckets == [[0, 1], [2]]
    for r in range(2):
        for v, x in enumerate(red.views()[r]):
            L = red.loc[v]
            assert np.shares_memory(x, red.flat[r][L.bucket]) and x.size == numels[v]


def test_planted_rebuild_mistakes_are_caught(monkeypatch):
    real = OR.Reducer.rebuild_buckets

    def reversed_order(self, cap=None):
        self.last_ready_order = self.last_ready_order[::-1]
        return real(self, cap)
    monkeypatch.setattr(OR.Reducer, "rebuild_buckets", reversed_order)
    caught = 0
    for t in (test_printed_first_iteration_then_rebuild, test_rebuild_packs_in_ready_order_with_the_cap_rule,
              test_rebuilt_buckets_never_wait_on_a_later_gradient):
        try:
            t()
        except AssertionError:
            caught += 1
    assert caught >= 1
