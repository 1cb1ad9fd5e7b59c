"""Pins for the oracle's gradient_as_bucket_view mode: the gradients are the
narrowed views of the flat buckets ([TP] "Internal Design", backward pass;
[C30] "gradient_as_bucket_view"), the hook copies nothing, and the results are
those of the copying reducer."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import reducer as OR
from workloads import gen as WG
from test_oracle_reducer import round_to_f32

MiB = 1 << 20


def _fill(views, seed, dyadic=False):
    for r, row in enumerate(views):
        for v, x in enumerate(row):
            x[...] = WG.dyadic(seed + 31 * r + v, x.size) if dyadic else \
                (np.random.default_rng(seed + 31 * r + v).standard_normal(x.size) * 1e-3).astype(np.float32)


def test_views_alias_the_flat_buckets_in_locator_order():
    numels = [5, 7, 3, 11, 2]
    red = OR.Reducer(numels, 3, 4 * 12, gradient_as_bucket_view=True)
    views = red.views()
    for r in range(3):
        for b, members in enumerate(red.buckets):
            off = 0
            for v in members:
                L = red.loc[v]
                assert (L.bucket, L.offset) == (b, off)
                assert np.shares_memory(views[r][v], red.flat[r][b])
                views[r][v][...] = 100 * r + v
                assert np.all(red.flat[r][b][off:off + numels[v]] == 100 * r + v)
                off += numels[v]
            assert off == red.flat[r][b].size            # the views tile the bucket


@pytest.mark.parametrize("seed", range(12))
def test_same_bits_as_the_copying_reducer(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 25))
    numels = WG.random_numels(seed, P, 1, 300)
    R = int(rng.integers(1, 9))
    cap = int(rng.integers(0, 4 * sum(numels)))
    order = WG.permutation(seed, P)
    a = OR.Reducer(numels, R, cap, gradient_as_bucket_view=True)
    _fill(a.views(), seed)
    local = [[x.copy() for x in row] for row in a.views()]
    b = OR.Reducer(numels, R, cap)
    g = [[x.copy() for x in row] for row in local]
    b.bind(g)
    a.sync(order)
    b.sync(order)
    assert a.launch_log == b.launch_log
    for r in range(R):
        for v in range(P):
            assert np.array_equal(a.views()[r][v].view(np.uint32), g[r][v].view(np.uint32))


def test_exact_rounded_mean_on_dyadic_inputs():
    numels = [9, 1, 40]
    R = 3
    red = OR.Reducer(numels, R, 0, gradient_as_bucket_view=True)
    _fill(red.views(), 7, dyadic=True)
    local = [[x.copy() for x in row] for row in red.views()]
    red.sync()
    for v, n in enumerate(numels):
        for i in range(n):
            want = round_to_f32(sum(Fraction(float(local[r][v][i])) for r in range(R)) / R)
            for r in range(R):
                assert red.views()[r][v][i].view(np.uint32) == want.view(np.uint32)


def test_no_sync_in_view_mode_matches_copy_mode():
    numels = [12, 30, 5]
    R, k = 4, 3
    steps = [[[WG.dyadic(t * 100 + r * 10 + v, n) for v, n in enumerate(numels)] for r in range(R)]
             for t in range(k)]
    a = OR.Reducer(numels, R, 4 * 20, gradient_as_bucket_view=True)
    b = OR.Reducer(numels, R, 4 * 20)
    g = [[np.zeros(n, np.float32) for n in numels] for _ in range(R)]
    b.bind(g)
    for red in (a, b):
        red.set_sync(False)
        for t in range(k):
            if t == k - 1:
                red.set_sync(True)
            red.no_sync_accumulate(steps[t], first=(t == 0))
            red.sync()
    for r in range(R):
        for v in range(len(numels)):
            assert np.array_equal(a.views()[r][v], g[r][v])


def test_planted_copy_instead_of_view_is_caught(monkeypatch):
    real_init = OR.Reducer.__init__

    def copying_views(self, *args, **kw):
        real_init(self, *args, **kw)
        if self.as_view:
            self.grads = [[x.copy() for x in row] for row in self.grads]
    monkeypatch.setattr(OR.Reducer, "__init__", copying_views)
    with pytest.raises(AssertionError):
        test_views_alias_the_flat_buckets_in_locator_order()
    caught = 0
    for seed in range(6):
        try:
            test_same_bits_as_the_copying_reducer(seed)
        except AssertionError:
            caught += 1
    assert caught >= 1
