"""Randomized GPU parity: seeded configurations that mix the replica count
(templated and generic-R kernels), ragged and empty tensors, bucket caps, the
fused, staged and bucket-view modes, capped launch grids, workgroups per CU,
used flags and permuted hook orders. Every replica's every gradient must equal the oracle's
bit for bit, over two iterations with fresh inputs."""
import numpy as np
import pytest
import torch

import ddp_bucketed_gradient_amd as D
from gpu_util import require_gpu, say, alloc_grads, fill_from_host, snapshot, assert_bits_equal
from oracle import reducer as OR
from workloads import gen as WG

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _config(seed):
    rng = np.random.default_rng(1000 + seed)
    P = int(rng.integers(1, 25))
    numels = [int(x) for x in rng.choice([0, 1, 3, 4, 5, 63, 64, 1000, 4096, 8191, 8192, 8193, 12289, 30001],
                                         size=P)]
    R = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 17, 20]))
    cap = int(rng.integers(0, 4 * max(sum(numels), 1) + 1))
    mode = str(rng.choice(["fused", "staged", "view"]))
    blocks = int(rng.choice([0, 0, 1, 3]))
    with_flags = bool(rng.integers(0, 2))
    wg = int(rng.choice([0, 1, 1, 2]))            # reduction workgroups per CU
    return rng, numels, R, cap, mode, blocks, with_flags, wg


@pytest.mark.parametrize("seed", range(100))
def test_random_configuration(seed):
    rng, numels, R, cap, mode, blocks, with_flags, wg = _config(seed)
    P = len(numels)
    say(f"random seed={seed} P={P} R={R} cap={cap} mode={mode} blocks={blocks} flags={with_flags} wg={wg}")
    red = D.Reducer([(n,) for n in numels], R, cap)
    view = mode == "view"
    orc = OR.Reducer(numels, R, cap, gradient_as_bucket_view=view)
    if view:
        grads = red.bind_bucket_views()
        grads = [[g.view(-1) for g in row] for row in grads]
        og = orc.views()
    else:
        grads = alloc_grads(numels, R)
        red.bind(grads, mode=D.MODE_STAGED if mode == "staged" else D.MODE_FUSED)
        og = [[np.zeros(n, np.float32) for n in numels] for _ in range(R)]
        orc.bind(og)
    red.set_launch_blocks(blocks)
    red.set_workgroups_per_cu(wg)
    for it in range(2):
        host = [[WG.normal(WG.seed_of(9, r, v, (seed * 2 + it) % 100), n).numpy() for v, n in enumerate(numels)]
                for r in range(R)]
        fill_from_host(grads, host)
        for r in range(R):
            for v in range(P):
                og[r][v][...] = host[r][v]
        used = (rng.random((R, P)) < 0.6) if with_flags else None
        G = np.ones(P, bool) if used is None else used.any(axis=0)
        order = [v for v in rng.permutation(P).tolist() if G[v]]
        if used is not None:
            red.set_local_used(used)
            orc.set_local_used(used)
        n_before = len(orc.launch_log)
        red.sync(order)
        orc.sync(order)
        got = snapshot(grads)
        assert red.launch_log() == orc.launch_log[n_before:]
        for v in range(P):
            for r in range(R):
                assert_bits_equal(got[v][r], og[r][v], f"seed={seed} it={it} v={v} r={r}")
    red.close()


def _sync_step_config(seed):
    rng = np.random.default_rng(5000 + seed)
    P = int(rng.integers(1, 16))
    numels = [int(x) for x in rng.choice([0, 1, 3, 4, 5, 64, 1000, 4096, 8191, 8192, 8193, 12289],
                                         size=P)]
    R = int(rng.choice([1, 2, 3, 4, 8, 15, 16, 17, 20, 33]))
    cap = int(rng.integers(0, 4 * max(sum(numels), 1) + 1))
    mode = str(rng.choice(["fused", "fused", "view", "staged"]))
    bf16 = bool(rng.integers(0, 2))
    k_before = int(rng.integers(0, 3))             # local steps before the synchronising one
    nulls = bool(rng.integers(0, 2))
    with_flags = rng.random() < 0.25
    blocks = int(rng.choice([0, 0, 0, 2]))
    wg = int(rng.choice([0, 1, 1, 2]))
    return rng, numels, R, cap, mode, bf16, k_before, nulls, with_flags, blocks, wg


@pytest.mark.parametrize("seed", range(40))
def test_random_sync_step(seed):
    """The synchronising micro-step fused into the reduction (set_sync_step)
    against the oracle's accumulate-then-sync, on seeded configurations: one,
    two or three chunks of replicas, bf16 and fp32 steps, first and later
    steps, missing steps, every mode, used flags, capped grids."""
    rng, numels, R, cap, mode, bf16, k_before, nulls, with_flags, blocks, wg = _sync_step_config(seed)
    P = len(numels)
    dtype = torch.bfloat16 if bf16 else torch.float32
    say(f"random sync step seed={seed} P={P} R={R} cap={cap} mode={mode} bf16={bf16} k={k_before} "
        f"nulls={nulls} flags={with_flags} blocks={blocks} wg={wg}")
    red = D.Reducer([(n,) for n in numels], R, cap)
    view = mode == "view"
    orc = OR.Reducer(numels, R, cap, gradient_as_bucket_view=view)
    if view:
        grads = [[g.view(-1) for g in row] for row in red.bind_bucket_views()]
        og = orc.views()
    else:
        grads = alloc_grads(numels, R)
        red.bind(grads, mode=D.MODE_STAGED if mode == "staged" else D.MODE_FUSED)
        og = [[np.zeros(n, np.float32) for n in numels] for _ in range(R)]
        orc.bind(og)
    red.set_launch_blocks(blocks)
    red.set_workgroups_per_cu(wg)
    init = [[WG.normal(WG.seed_of(15, r, v, seed % 100), n).numpy() for v, n in enumerate(numels)] for r in range(R)]
    fill_from_host(grads, init)
    for r in range(R):
        for v in range(P):
            og[r][v][...] = init[r][v]

    def steps(t):
        host, dev = [], []
        for r in range(R):
            hrow, drow = [], []
            for v, n in enumerate(numels):
                if nulls and rng.random() < 0.25:
                    hrow.append(None)
                    drow.append(None)
                    continue
                x = WG.normal(WG.seed_of(16, r, v, (seed * 3 + t) % 100), n)
                if bf16:
                    xb = x.to(torch.bfloat16)
                    hrow.append(xb.view(torch.int16).numpy().view(np.uint16).copy())
                    drow.append(xb.cuda())
                else:
                    hrow.append(x.numpy().copy())
                    drow.append(x.cuda())
            host.append(hrow)
            dev.append(drow)
        return host, dev

    keep = []
    red.set_sync(False)
    orc.set_sync(False)
    for t in range(k_before):
        hs, ds = steps(t)
        keep.append(ds)
        red.no_sync_accumulate(ds, first_step=(t == 0))
        orc.no_sync_accumulate(hs, first=(t == 0))
    red.set_sync(True)
    orc.set_sync(True)
    used = None
    if with_flags:
        used = rng.random((R, P)) < 0.7
        red.set_local_used(used)
        orc.set_local_used(used)
    hs, ds = steps(k_before)
    keep.append(ds)
    first = k_before == 0
    red.set_sync_step(ds if seed % 2 else red.step_table(ds), first_step=first)
    orc.no_sync_accumulate(hs, first=first)
    G = np.ones(P, bool) if used is None else used.any(axis=0)
    order = [v for v in rng.permutation(P).tolist() if G[v]]
    n_before = len(orc.launch_log)
    red.sync(order)
    orc.sync(order)
    got = snapshot(grads)
    assert red.launch_log() == orc.launch_log[n_before:]
    for v in range(P):
        for r in range(R):
            assert_bits_equal(got[v][r], og[r][v], f"sync step seed={seed} v={v} r={r}")
    red.close()
