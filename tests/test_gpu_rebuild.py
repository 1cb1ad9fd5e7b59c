"""GPU parity after a ready-order bucket rebuild, in the copying mode and in
the bucket-view mode, against the oracle's rebuild on the same inputs."""
import pytest
import torch

import ddp_bucketed_gradient_amd as D
from gpu_util import require_gpu, alloc_grads, fill_from_host, snapshot, assert_bits_equal
from oracle import reducer as OR
from workloads import gen as WG

pytestmark = pytest.mark.gpu

NUMELS = [1, 3, 4097, 8193, 12345, 64, 20000, 5, 70000, 2, 777, 4096]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _host(seed, R):
    return [[WG.normal(WG.seed_of(6, r, v, seed), n).numpy() for v, n in enumerate(NUMELS)] for r in range(R)]


def test_rebuild_then_parity_copying_mode():
    R = 4
    order = WG.permutation(5, len(NUMELS))           # not the reverse-index order
    red = D.Reducer([(n,) for n in NUMELS], R, 1 << 62)   # first iteration: one bucket
    grads = alloc_grads(NUMELS, R)
    red.bind(grads)
    orc = OR.Reducer(NUMELS, R, 1 << 62)
    host0 = _host(0, R)
    fill_from_host(grads, host0)
    orc.bind([[h.copy() for h in row] for row in host0])
    red.sync(order)
    orc.sync(order)
    red.rebuild_buckets(4 * 15000)
    orc.rebuild_buckets(4 * 15000)
    assert red.buckets() == orc.buckets
    red.bind(grads)
    host1 = _host(1, R)
    fill_from_host(grads, host1)
    for r in range(R):
        for v in range(len(NUMELS)):
            orc.grads[r][v][...] = host1[r][v]
    orc.launch_log.clear()
    red.sync(order)
    orc.sync(order)
    got = snapshot(grads)
    assert red.launch_log() == orc.launch_log
    for v in range(len(NUMELS)):
        for r in range(R):
            assert_bits_equal(got[v][r], orc.grads[r][v], f"v={v} r={r}")


def test_rebuild_then_parity_bucket_view_mode():
    R = 3
    order = WG.permutation(9, len(NUMELS))
    red = D.Reducer([(n,) for n in NUMELS], R, 4 * 9000)
    views = red.bind_bucket_views()
    orc = OR.Reducer(NUMELS, R, 4 * 9000, gradient_as_bucket_view=True)
    red.sync(order)
    orc.sync(order)
    red.rebuild_buckets()
    orc.rebuild_buckets()
    views = red.bind_bucket_views()                  # new layout, new views
    host = _host(2, R)
    for r in range(R):
        for v in range(len(NUMELS)):
            views[r][v].copy_(torch.from_numpy(host[r][v]))
            orc.views()[r][v][...] = host[r][v]
    orc.launch_log.clear()
    red.sync(order)
    orc.sync(order)
    torch.cuda.synchronize()
    assert red.launch_log() == orc.launch_log
    for r in range(R):
        for v in range(len(NUMELS)):
            assert_bits_equal(views[r][v].cpu().numpy(), orc.views()[r][v], f"r={r} v={v}")
