"""GPU parity with unused parameters: the HIP path against the oracle, bit for
bit, in the fused, staged and bucket-view modes, with per-replica used flags
(some variables used by no replica, some by only a few), flags OR-ed over
no_sync micro-steps, and every variable unused."""
import numpy as np
import pytest
import torch

import ddp_bucketed_gradient_amd as D
from gpu_util import require_gpu, say, alloc_grads, fill_from_host, snapshot, assert_bits_equal
from oracle import reducer as OR
from workloads import gen as WG

pytestmark = pytest.mark.gpu

NUMELS = [1, 3, 4097, 8193, 12345, 64, 20000, 5, 70000, 2, 777, 4096, 0, 16384]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _host(seed, R, numels=NUMELS):
    return [[WG.normal(WG.seed_of(7, r, v, seed), n).numpy() for v, n in enumerate(numels)] for r in range(R)]


def _flags(seed, R, P):
    rng = np.random.default_rng(seed)
    used = rng.random((R, P)) < 0.5
    used[:, 0] = False                    # used by no replica
    used[:, 1] = True                     # used by every replica
    used[0, 2] = True                     # used by replica 0 only
    used[1:, 2] = False
    return used


@pytest.mark.parametrize("R", [2, 3, 8, 20, 24, 64])
@pytest.mark.parametrize("mode", [D.MODE_FUSED, D.MODE_STAGED])
def test_unused_parity_copy_modes(R, mode):
    P = len(NUMELS)
    cap = 4 * 15000
    say(f"unused copy modes R={R} mode={mode}")
    red = D.Reducer([(n,) for n in NUMELS], R, cap)
    grads = alloc_grads(NUMELS, R)
    red.bind(grads, mode=mode)
    orc = OR.Reducer(NUMELS, R, cap)
    og = [[np.zeros(n, np.float32) for n in NUMELS] for _ in range(R)]
    orc.bind(og)
    for it in range(3):                   # flags, then none, then other flags
        host = _host((10 * R + it) % 100, R)
        fill_from_host(grads, host)
        for r in range(R):
            for v in range(P):
                og[r][v][...] = host[r][v]
        used = None if it == 1 else _flags(R * 100 + it + mode, R, P)
        G = np.ones(P, bool) if used is None else used.any(axis=0)
        order = [v for v in WG.permutation(R + it, P) if G[v]]
        if used is not None:
            red.set_local_used(used)
            orc.set_local_used(used)
        orc.launch_log.clear()
        red.sync(order)
        orc.sync(order)
        got = snapshot(grads)
        assert red.launch_log() == orc.launch_log
        for v in range(P):
            for r in range(R):
                assert_bits_equal(got[v][r], og[r][v], f"it={it} v={v} r={r}")


@pytest.mark.parametrize("R", [3, 8])
def test_unused_parity_bucket_views(R):
    P = len(NUMELS)
    cap = 4 * 9000
    say(f"unused bucket views R={R}")
    red = D.Reducer([(n,) for n in NUMELS], R, cap)
    views = red.bind_bucket_views()
    orc = OR.Reducer(NUMELS, R, cap, gradient_as_bucket_view=True)
    for it in range(2):
        host = _host(50 + it, R)
        for r in range(R):
            for v in range(P):
                views[r][v].copy_(torch.from_numpy(host[r][v]))
                orc.views()[r][v][...] = host[r][v]
        used = _flags(R + it, R, P)
        order = [v for v in WG.permutation(R * 3 + it, P) if used[:, v].any()]
        red.set_local_used(used)
        orc.set_local_used(used)
        orc.launch_log.clear()
        red.sync(order)
        orc.sync(order)
        torch.cuda.synchronize()
        assert red.launch_log() == orc.launch_log
        for r in range(R):
            for v in range(P):
                assert_bits_equal(views[r][v].cpu().numpy(), orc.views()[r][v], f"it={it} r={r} v={v}")


def test_unused_flags_or_over_no_sync_steps():
    numels = NUMELS
    P, R, k = len(numels), 4, 3
    say("unused no_sync OR")
    red = D.Reducer([(n,) for n in numels], R, 4 * 20000)
    grads = alloc_grads(numels, R)
    red.bind(grads)
    orc = OR.Reducer(numels, R, 4 * 20000)
    og = [[np.zeros(n, np.float32) for n in numels] for _ in range(R)]
    orc.bind(og)
    rng = np.random.default_rng(3)
    used_t = [rng.random((R, P)) < 0.4 for _ in range(k)]
    for u in used_t:
        u[:, 0] = False                   # never used in any micro-step
    dsteps, hsteps = [], []
    for t in range(k):
        drow, hrow = [], []
        for r in range(R):
            d, h = [], []
            for v, n in enumerate(numels):
                if used_t[t][r, v]:
                    x = WG.normal(WG.seed_of(8, r, v, t), n).numpy()
                    d.append(torch.from_numpy(x).cuda())
                    h.append(x)
                else:
                    d.append(None)
                    h.append(None)
            drow.append(d)
            hrow.append(h)
        dsteps.append(drow)
        hsteps.append(hrow)
    red.set_sync(False)
    orc.set_sync(False)
    for t in range(k):
        if t == k - 1:
            red.set_sync(True)
            orc.set_sync(True)
        red.set_local_used(used_t[t])
        orc.set_local_used(used_t[t])
        red.no_sync_accumulate(dsteps[t], first_step=(t == 0))
        orc.no_sync_accumulate(hsteps[t], first=(t == 0))
        G = orc.globally_used()
        order = [v for v in range(P - 1, -1, -1) if G[v]]
        red.sync(order)
        orc.sync(order)
    got = snapshot(grads)
    for v in range(P):
        for r in range(R):
            assert_bits_equal(got[v][r], og[r][v], f"v={v} r={r}")


@pytest.mark.parametrize("mode", [D.MODE_FUSED, D.MODE_STAGED])
def test_every_variable_unused(mode):
    R = 3
    say(f"all unused mode={mode}")
    red = D.Reducer([(n,) for n in NUMELS], R, 4 * 10000)
    grads = alloc_grads(NUMELS, R)
    red.bind(grads, mode=mode)
    host = _host(99, R)
    fill_from_host(grads, host)
    red.set_local_used(np.zeros((R, len(NUMELS)), bool))
    red.finalize()
    got = snapshot(grads)
    assert [b for b, _ in red.launch_log()] == list(range(red.num_buckets))
    for v in range(len(NUMELS)):
        for r in range(R):
            assert_bits_equal(got[v][r], host[r][v], f"v={v} r={r}")   # untouched


@pytest.mark.parametrize("mode", [D.MODE_FUSED, D.MODE_STAGED])
def test_reset_after_failed_iteration_drops_flags(mode):
    """An iteration with used flags fails (half of its hooks fire, finalize
    refuses), the reducer is reset, and the next synchronisation runs with
    other flags: its result is the oracle's under the new flags alone (the
    failed iteration's flags are not OR-ed in), bit for bit."""
    R, P, cap = 4, len(NUMELS), 4 * 15000
    say(f"reset after a failed iteration with flags, mode={mode}")
    red = D.Reducer([(n,) for n in NUMELS], R, cap)
    grads = alloc_grads(NUMELS, R)
    red.bind(grads, mode=mode)
    orc = OR.Reducer(NUMELS, R, cap)
    og = [[np.zeros(n, np.float32) for n in NUMELS] for _ in range(R)]
    orc.bind(og)
    host = _host(31, R)
    fill_from_host(grads, host)
    for r in range(R):
        for v in range(P):
            og[r][v][...] = host[r][v]
    used_a = _flags(301 + mode, R, P)
    red.set_local_used(used_a)
    orc.set_local_used(used_a)
    first = [v for v in WG.permutation(32, P) if used_a.any(axis=0)[v]]
    first = first[:len(first) // 2]
    for v in first:
        red.mark_ready(v)
        orc.mark_ready(v)
    with pytest.raises(D.DdpbError) as e:
        red.finalize()
    assert e.value.code == D.E_INCOMPLETE
    with pytest.raises(OR.ReductionIncomplete):
        orc.finalize()
    red.reset()
    orc.reset()
    torch.cuda.synchronize()
    host = _host(33, R)
    fill_from_host(grads, host)
    for r in range(R):
        for v in range(P):
            og[r][v][...] = host[r][v]
    used_b = _flags(302 + mode, R, P)
    used_b[:, 0] = True                   # used by every replica now (unused by all before)
    G = used_b.any(axis=0)
    order = [v for v in WG.permutation(34, P) if G[v]]
    red.set_local_used(used_b)
    orc.set_local_used(used_b)
    orc.launch_log.clear()
    red.sync(order)
    orc.sync(order)
    got = snapshot(grads)
    assert red.launch_log() == orc.launch_log
    for v in range(P):
        for r in range(R):
            assert_bits_equal(got[v][r], og[r][v], f"after reset v={v} r={r}")
    red.close()
