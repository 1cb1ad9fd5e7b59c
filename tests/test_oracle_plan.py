"""Pins for the oracle's bucket planner and locator.

Each test checks the oracle against something other than itself: the layouts
the pages print, invariants of the assignment rule checked by brute force, and
planted mistakes that must be caught.
"""
import itertools

import numpy as np
import pytest

from conftest import load_golden
from oracle import plan as OP
from workloads import shapes as WS, gen as WG

MiB = 1 << 20


def _bytes(buckets, numels, es=4):
    return [sum(numels[v] for v in b) * es for b in buckets]


# --- printed worked examples -------------------------------------------------

def test_printed_layouts_param_granularity():
    g = load_golden("c30_param_granularity.json")
    for row in g["rows"]:
        numels = [row["param_bytes"] // 4] * row["param_count"]
        assert sum(numels) * 4 == g["payload_bytes"]
        bk = OP.compute_bucket_assignment_by_size(numels, 4, row["cap_bytes"])
        assert len(bk) == row["buckets"], row["name"]
        assert all(len(b) == row["params_per_bucket"] for b in bk), row["name"]
        assert all(x == row["bucket_bytes"] for x in _bytes(bk, numels)), row["name"]


def test_cap_is_not_a_ceiling():
    g = load_golden("c30_cap_not_ceiling.json")
    numels = [g["param_bytes"] // 4]
    bk = OP.compute_bucket_assignment_by_size(numels, 4, g["cap_bytes"])
    assert _bytes(bk, numels) == [g["bucket_bytes"]]
    # and between smaller neighbours it still stays whole
    numels = [MiB // 4, g["param_bytes"] // 4, MiB // 4]
    bk = OP.compute_bucket_assignment_by_size(numels, 4, g["cap_bytes"])
    assert all(len(set(b)) == len(b) for b in bk)
    assert sorted(v for b in bk for v in b) == [0, 1, 2]
    assert _bytes(bk, numels)[0] == g["param_bytes"] + MiB   # v2 then v1 closes at 9 MiB


def test_single_bucket_bytes():
    g = load_golden("c30_single_bucket.json")
    numels = [MiB] * 12
    bk = OP.compute_bucket_assignment_by_size(numels, 4, 1 << 62)
    assert _bytes(bk, numels) == [g["bucket_bytes"]]


def test_bucket0_holds_last_defined_parameters():
    # the first bucket to fill holds the final layers ([Li] "Why reverse order")
    for params in (WS.resnet50(), WS.bert_large(), WS.mlp()):
        n = WS.numels(params)
        bk = OP.compute_bucket_assignment_by_size(n, 4, 25 * MiB)
        assert bk[0][0] == len(n) - 1
        assert bk[-1][-1] == 0


# --- invariants of the rule, brute force on random shape lists ---------------

@pytest.mark.parametrize("seed", range(40))
def test_assignment_invariants_random(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 40))
    numels = WG.random_numels(seed, P, 1, 3000)
    total = sum(numels) * 4
    cap = int(rng.integers(0, total + 100))
    bk = OP.compute_bucket_assignment_by_size(numels, 4, cap)
    # concatenation is exactly P-1 .. 0
    assert [v for b in bk for v in b] == list(range(P - 1, -1, -1))
    sizes = _bytes(bk, numels)
    for i, b in enumerate(bk):
        if i < len(bk) - 1:
            assert sizes[i] >= cap                      # closed because it reached the cap
        if len(b) > 1:
            assert sizes[i] - numels[b[-1]] * 4 < cap   # it did not reach it one tensor earlier
    # locator offsets are prefix sums inside each bucket
    loc = OP.locators(bk, numels)
    for bi, b in enumerate(bk):
        off = 0
        for i, v in enumerate(b):
            assert loc[v] == OP.Locator(bi, i, off, numels[v])
            off += numels[v]


def test_cap_zero_is_per_tensor_and_huge_cap_is_one_bucket():
    numels = WS.numels(WS.bert_large())
    assert len(OP.compute_bucket_assignment_by_size(numels, 4, 0)) == len(numels)
    assert len(OP.compute_bucket_assignment_by_size(numels, 4, sum(numels) * 4 + 1)) == 1
    # exactly the total: closes on the last tensor, still one bucket
    assert len(OP.compute_bucket_assignment_by_size(numels, 4, sum(numels) * 4)) == 1


def test_empty_model():
    assert OP.compute_bucket_assignment_by_size([], 4, 25 * MiB) == []


def test_bruteforce_against_exhaustive_definition():
    # For tiny lists, enumerate every way of cutting P-1..0 into consecutive
    # groups and keep the one that satisfies the rule's two conditions; it
    # must be unique and equal the oracle's.
    rng = np.random.default_rng(7)
    for _ in range(200):
        P = int(rng.integers(1, 8))
        numels = [int(x) for x in rng.integers(1, 20, size=P)]
        cap = int(rng.integers(0, 60)) * 4
        order = list(range(P - 1, -1, -1))
        found = []
        for cuts in itertools.product([0, 1], repeat=P - 1):
            groups, cur = [], [order[0]]
            for c, v in zip(cuts, order[1:]):
                if c:
                    groups.append(cur)
                    cur = [v]
                else:
                    cur.append(v)
            groups.append(cur)
            ok = True
            for gi, g in enumerate(groups):
                sz = sum(numels[v] for v in g) * 4
                before_last = sz - numels[g[-1]] * 4
                if gi < len(groups) - 1 and sz < cap:
                    ok = False           # a closed bucket must have reached the cap
                if len(g) > 1 and before_last >= cap:
                    ok = False           # it would have closed one tensor earlier
            if ok:
                found.append(groups)
        assert len(found) == 1
        assert found[0] == OP.compute_bucket_assignment_by_size(numels, 4, cap)


# --- derived workload facts ----------------------------------------------------

def test_workload_totals_and_bucket_counts():
    cases = [
        (WS.resnet50(), 161, 25_557_032, {25: 4}),
        (WS.bert_large(), 391, 335_141_888,
         {0: 391, 1: 147, 5: 97, 10: 73, 25: 37, 50: 21, 100: 12, 200: 6}),
        (WS.bert_base(), 199, 109_482_240, {25: 13}),
        (WS.mlp(), 96, 805_552_128, {25: 48}),
        (WS.linear10(), 2, 110, {25: 1}),
    ]
    for params, P, total, caps in cases:
        n = WS.numels(params)
        assert len(n) == P and sum(n) == total
        for cap_mib, B in caps.items():
            assert len(OP.compute_bucket_assignment_by_size(n, 4, cap_mib * MiB)) == B, (P, cap_mib)
    n = WS.numels(WS.linear10())
    bk = OP.compute_bucket_assignment_by_size(n, 4, 25 * MiB)
    loc = OP.locators(bk, n)
    assert bk == [[1, 0]]
    assert loc[1] == OP.Locator(0, 0, 0, 10) and loc[0] == OP.Locator(0, 1, 10, 100)


# --- planted mistakes must be caught by the pins above -------------------------

def _strict_greater(numels, es, cap):
    out, cur, size = [], [], 0
    for v in range(len(numels) - 1, -1, -1):
        cur.append(v)
        size += numels[v] * es
        if size > cap:
            out.append(cur)
            cur, size = [], 0
    if cur:
        out.append(cur)
    return out


def _forward_order(numels, es, cap):
    out, cur, size = [], [], 0
    for v in range(len(numels)):
        cur.append(v)
        size += numels[v] * es
        if size >= cap:
            out.append(cur)
            cur, size = [], 0
    if cur:
        out.append(cur)
    return out


_REAL_PLAN = OP.compute_bucket_assignment_by_size


def _drops_tail(numels, es, cap):
    return [b for b in _REAL_PLAN(numels, es, cap)
            if sum(numels[v] for v in b) * es >= cap]


@pytest.mark.parametrize("mutant", [_strict_greater, _forward_order, _drops_tail])
def test_planted_planner_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(OP, "compute_bucket_assignment_by_size", mutant)
    failures = 0
    for t in (test_printed_layouts_param_granularity, test_bucket0_holds_last_defined_parameters,
              test_workload_totals_and_bucket_counts, test_cap_zero_is_per_tensor_and_huge_cap_is_one_bucket):
        try:
            t()
        except AssertionError:
            failures += 1
    assert failures >= 1
