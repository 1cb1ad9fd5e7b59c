"""CPU tests of the native ready-order rebuild (host-only build) against the
oracle: same new plan, same launches afterwards, documented errors."""
import os

import numpy as np
import pytest

import ddp_bucketed_gradient_amd as D
from ddp_bucketed_gradient_amd import _abi
from oracle import reducer as OR
from workloads import gen as WG

MiB = 1 << 20


@pytest.fixture(scope="module")
def host():
    if not os.path.exists(D.HOSTONLY_LIB):
        from ddp_bucketed_gradient_amd import build
        build.build_hostonly()
    return D.Lib(D.HOSTONLY_LIB)


def _bind(red):
    red.bind_ptrs([0x1000 + 16 * i for i in range(red.R * red.P)], side_streams=[0])


@pytest.mark.parametrize("seed", range(15))
def test_rebuild_matches_oracle(host, seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 50))
    numels = WG.random_numels(seed, P, 0, 400)
    cap0 = int(rng.integers(0, 4 * sum(numels) + 1))
    cap1 = int(rng.integers(0, 4 * sum(numels) + 1))
    order = WG.permutation(seed, P)
    red = D.Reducer([(n,) for n in numels], 2, cap0, lib=host)
    orc = OR.Reducer(numels, 2, cap0)
    orc.bind([[np.zeros(n, np.float32) for n in numels] for _ in range(2)])
    _bind(red)
    red.sync(order)
    orc.sync(order)
    assert red.ready_order() == order == orc.last_ready_order
    red.rebuild_buckets(cap1)
    orc.rebuild_buckets(cap1)
    assert red.buckets() == orc.buckets
    for v in range(P):
        L = orc.loc[v]
        assert red.locator(v) == (L.bucket, L.intra, L.offset, L.length)
    with pytest.raises(D.DdpbError) as e:
        red.mark_ready(order[0])                    # must be bound again
    assert e.value.code == _abi.E_STATE
    _bind(red)
    order2 = WG.permutation(seed + 100, P)
    orc.launch_log.clear()
    red.sync(order2)
    orc.sync(order2)
    assert red.launch_log() == orc.launch_log


def test_printed_first_iteration_then_rebuild_native(host):
    numels = [MiB] * 12
    order = list(range(11, -1, -1))
    for cap, nb in [(4 * MiB, 12), (16 * MiB, 3), (64 * MiB, 1)]:
        red = D.Reducer([(n,) for n in numels], 2, 1 << 62, lib=host)
        assert red.bucket_bytes() == [50331648]
        _bind(red)
        red.sync(order)
        red.rebuild_buckets(cap)
        assert red.num_buckets == nb


def test_rebuild_errors(host):
    red = D.Reducer([(4,), (4,)], 2, 0, lib=host)
    with pytest.raises(D.DdpbError) as e:
        red.rebuild_buckets()                       # nothing learned yet
    assert e.value.code == _abi.E_STATE
    _bind(red)
    red.mark_ready(1)
    with pytest.raises(D.DdpbError) as e:
        red.rebuild_buckets()                       # iteration in progress
    assert e.value.code == _abi.E_INCOMPLETE


def test_rebind_starts_the_launch_history_afresh(host):
    """After a rebuild and a new bind the old plan's launches are gone: the log
    is empty and timing queries for iterations of the earlier binding fail
    with an index error rather than reading the new binding's resources."""
    numels = [5, 7, 3, 9]
    red = D.Reducer([(n,) for n in numels], 2, 4 * 8, lib=host)
    _bind(red)
    red.sync([3, 2, 1, 0])
    assert red.launch_log() != []
    red.rebuild_buckets(0)
    assert red.launch_log() == []
    _bind(red)
    assert red.launch_log() == []
    with pytest.raises(D.DdpbError) as e:
        red.launch_times_ms(0)
    assert e.value.code == _abi.E_INDEX
