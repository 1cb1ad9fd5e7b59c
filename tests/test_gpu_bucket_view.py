"""GPU parity of gradient_as_bucket_view: gradients are views into one flat
storage per replica; the reduction walks each bucket's flat range. Compared
bit for bit with the oracle's bucket-view mode on the same inputs."""
import numpy as np
import pytest
import torch

import ddp_bucketed_gradient_amd as D
from gpu_util import require_gpu, assert_bits_equal
from oracle import reducer as OR
from workloads import gen as WG

pytestmark = pytest.mark.gpu

RAGGED = [1, 3, 4, 5, 63, 64, 65, 255, 1000, 4095, 4096, 4097, 8191, 8193, 12345, 20000, 2, 777, 70000]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _host(seed, numels, R):
    return [[WG.normal(WG.seed_of(8, r, v, seed), n).numpy() for v, n in enumerate(numels)] for r in range(R)]


@pytest.mark.parametrize("R", [1, 3, 8])
def test_bucket_view_parity(R):
    numels = RAGGED
    cap = 4 * 11000
    order = WG.permutation(R + 100, len(numels))
    red = D.Reducer([(n,) for n in numels], R, cap)
    views = red.bind_bucket_views()
    orc = OR.Reducer(numels, R, cap, gradient_as_bucket_view=True)
    for it in range(2):
        host = _host(it, numels, R)
        for r in range(R):
            for v in range(len(numels)):
                views[r][v].copy_(torch.from_numpy(host[r][v]))
                orc.views()[r][v][...] = host[r][v]
        orc.launch_log.clear()
        red.sync(order)
        orc.sync(order)
        torch.cuda.synchronize()
        assert red.launch_log() == orc.launch_log
        for r in range(R):
            for v in range(len(numels)):
                assert_bits_equal(views[r][v].cpu().numpy(), orc.views()[r][v], f"it={it} r={r} v={v}")


def test_bucket_view_no_sync_with_unaligned_views():
    """Views at odd element offsets (bucket members are packed without
    padding) take the scalar path of the accumulate kernel."""
    numels = [3, 4097, 5, 10000, 1]
    R, k = 4, 3
    red = D.Reducer([(n,) for n in numels], R, 4 * 20000)
    views = red.bind_bucket_views()
    assert any(red.view_offset(v) % 4 for v in range(len(numels)))
    orc = OR.Reducer(numels, R, 4 * 20000, gradient_as_bucket_view=True)
    steps = [[[WG.normal(WG.seed_of(8, r, v, 50 + t), n, "cuda").to(torch.bfloat16) for v, n in enumerate(numels)]
              for r in range(R)] for t in range(k)]
    red.set_sync(False)
    orc.set_sync(False)
    for t in range(k):
        if t == k - 1:
            red.set_sync(True)
            orc.set_sync(True)
        red.no_sync_accumulate(steps[t], first_step=(t == 0))
        hs = [[steps[t][r][v].view(torch.int16).cpu().numpy().view(np.uint16) for v in range(len(numels))]
              for r in range(R)]
        orc.no_sync_accumulate(hs, first=(t == 0))
        red.sync()
        orc.sync()
    torch.cuda.synchronize()
    for r in range(R):
        for v in range(len(numels)):
            assert_bits_equal(views[r][v].cpu().numpy(), orc.views()[r][v], f"r={r} v={v}")
