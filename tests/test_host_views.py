"""CPU tests of the gradient_as_bucket_view layout and binding through the C
ABI (host-only build): the view offsets follow the oracle's plan, and the
state machine behaves as in the copying mode."""
import os

import pytest

import ddp_bucketed_gradient_amd as D
from oracle import plan as OP
from oracle import reducer as OR
from workloads import shapes as WS, gen as WG

MiB = 1 << 20


@pytest.fixture(scope="module")
def host():
    if not os.path.exists(D.HOSTONLY_LIB):
        from ddp_bucketed_gradient_amd import build
        build.build_hostonly()
    return D.Lib(D.HOSTONLY_LIB)


def _expected_layout(numels, cap):
    """Each bucket's flat range starts on a 64-element boundary; a variable
    sits at its bucket's base plus its locator offset."""
    bk = OP.compute_bucket_assignment_by_size(numels, 4, cap)
    loc = OP.locators(bk, numels)
    sizes = OP.bucket_numels(bk, numels)
    bases, base = [], 0
    for n in sizes:
        bases.append(base)
        base += -(-n // 64) * 64
    return [bases[loc[v].bucket] + loc[v].offset for v in range(len(numels))], base


@pytest.mark.parametrize("numels,cap", [
    (WS.numels(WS.linear10()), 25 * MiB),
    (WS.numels(WS.resnet50()), 25 * MiB),
    (WS.numels(WS.bert_large()), 25 * MiB),
    (WG.random_numels(3, 50, 1, 3000), 4 * 5000),
    ([0, 5, 0, 7], 0),
])
def test_view_offsets_and_storage(host, numels, cap):
    red = D.Reducer([(n,) for n in numels], 2, cap, lib=host)
    offs, total = _expected_layout(numels, cap)
    assert host.view_storage_elems(red.h) == total
    assert [red.view_offset(v) for v in range(len(numels))] == offs
    # views never overlap and stay inside the storage
    spans = sorted((o, o + n) for o, n in zip(offs, numels) if n)
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    assert all(e <= total for _, e in spans)


def test_view_bind_runs_the_same_state_machine(host):
    numels = WG.random_numels(8, 30, 1, 200)
    cap = 4 * 300
    red = D.Reducer([(n,) for n in numels], 3, cap, lib=host)
    n = host.view_storage_elems(red.h)
    host.bind_bucket_views(red.h, [0x10000, 0x20000 + 256, 0x90000], n, 0, [0])
    orc = OR.Reducer(numels, 3, cap, gradient_as_bucket_view=True)
    for it in range(2):
        order = WG.permutation(it, len(numels))
        orc.launch_log.clear()
        orc.sync(order)
        red.sync(order)
        assert red.launch_log() == orc.launch_log


def test_view_bind_errors(host):
    red = D.Reducer([(10,), (20,)], 2, 0, lib=host)
    n = host.view_storage_elems(red.h)
    with pytest.raises(D.DdpbError):
        host.bind_bucket_views(red.h, [0x1000, 0x2000], n - 1, 0, [0])      # storage too small
    with pytest.raises(D.DdpbError):
        host.bind_bucket_views(red.h, [0x1000, 0], n, 0, [0])               # null storage
    with pytest.raises(D.DdpbError):
        host.bind_bucket_views(red.h, [0x1000, 0x2000], n, 0, [])           # no side stream
