"""The synchronising micro-step accumulated by the reduction itself
(ddpb_set_sync_step) against the oracle run as the pages describe it: every
local step accumulated into the gradients (no_sync), then the synchronisation.
Bit for bit, every replica, fused and bucket-view modes (one kernel per
bucket), staged mode and used flags (accumulation on the side stream, then the
usual reduction), bf16 and fp32 steps, first and later steps, replicas with
no step (NULL), power-of-two and other replica counts, the generic-R kernel."""
import numpy as np
import pytest
import torch

import ddp_bucketed_gradient_amd as D
from gpu_util import require_gpu, say, alloc_grads, fill_from_host, snapshot, assert_bits_equal
from oracle import reducer as OR
from workloads import gen as WG

pytestmark = pytest.mark.gpu

NUMELS = [1, 3, 4097, 8193, 12345, 64, 20000, 5, 70000, 2, 777, 4096, 0]

# name, R, cap bytes, mode, step dtype, micro-steps before the synchronising one, NULL steps, used flags
CASES = [
    ("fused_r3_bf16_add_nulls", 3, 4 * 15000, "fused", torch.bfloat16, 2, True, False),
    ("fused_r8_f32_first", 8, 4 * 15000, "fused", torch.float32, 0, False, False),
    ("fused_r16_bf16_add", 16, 4 * 40000, "fused", torch.bfloat16, 1, False, False),
    ("fused_r20_bf16_add", 20, 4 * 15000, "fused", torch.bfloat16, 1, True, False),
    ("fused_r2_f32_add_cap0", 2, 0, "fused", torch.float32, 1, False, False),
    ("view_r4_bf16_add_nulls", 4, 4 * 15000, "view", torch.bfloat16, 2, True, False),
    ("staged_r8_bf16_add", 8, 4 * 15000, "staged", torch.bfloat16, 1, True, False),
    ("fused_r8_bf16_add_used", 8, 4 * 15000, "fused", torch.bfloat16, 1, True, True),
    ("view_r3_f32_first_used", 3, 4 * 15000, "view", torch.float32, 0, True, True),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _steps(case_id, t, R, dtype, nulls, rng):
    """R x P step gradients of micro-step t (numpy for the oracle: float32, or
    uint16 bf16 bit patterns) and the device tensors (None where NULL)."""
    host, dev = [], []
    for r in range(R):
        hrow, drow = [], []
        for v, n in enumerate(NUMELS):
            if nulls and rng.random() < 0.2:
                hrow.append(None)
                drow.append(None)
                continue
            x = WG.normal(WG.seed_of(11, r, v, (case_id * 10 + t) % 100), n)
            if dtype == torch.bfloat16:
                xb = x.to(torch.bfloat16)
                hrow.append(xb.view(torch.int16).numpy().view(np.uint16).copy())
                drow.append(xb.cuda())
            else:
                hrow.append(x.numpy().copy())
                drow.append(x.cuda())
        host.append(hrow)
        dev.append(drow)
    return host, dev


@pytest.mark.parametrize("case", range(len(CASES)))
def test_sync_step_matches_accumulate_then_sync(case):
    name, R, cap, mode, dtype, k_before, nulls, with_flags = CASES[case]
    P = len(NUMELS)
    say(f"sync step case {name}")
    rng = np.random.default_rng(case)
    red = D.Reducer([(n,) for n in NUMELS], R, cap)
    orc = OR.Reducer(NUMELS, R, cap, gradient_as_bucket_view=(mode == "view"))
    if mode == "view":
        grads = [[g.view(-1) for g in row] for row in red.bind_bucket_views()]
        og = orc.views()
    else:
        grads = alloc_grads(NUMELS, R)
        red.bind(grads, mode=D.MODE_STAGED if mode == "staged" else D.MODE_FUSED)
        og = [[np.zeros(n, np.float32) for n in NUMELS] for _ in range(R)]
        orc.bind(og)
    init = [[WG.normal(WG.seed_of(12, r, v, case), n).numpy() for v, n in enumerate(NUMELS)] for r in range(R)]
    fill_from_host(grads, init)
    for r in range(R):
        for v in range(P):
            og[r][v][...] = init[r][v]
    keep = []
    red.set_sync(False)
    orc.set_sync(False)
    for t in range(k_before):                           # local steps inside no_sync
        hs, ds = _steps(case, t, R, dtype, nulls, rng)
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
    hs, ds = _steps(case, k_before, R, dtype, nulls, rng)   # the synchronising step
    keep.append(ds)
    first = k_before == 0
    red.set_sync_step(ds, first_step=first)
    orc.no_sync_accumulate(hs, first=first)
    G = np.ones(P, bool) if used is None else used.any(axis=0)
    order = [v for v in WG.permutation(60 + case, P) if G[v]]
    n_before = len(orc.launch_log)
    red.sync(order)
    orc.sync(order)
    got = snapshot(grads)
    assert red.launch_log() == orc.launch_log[n_before:]
    for v in range(P):
        for r in range(R):
            assert_bits_equal(got[v][r], og[r][v], f"{name} v={v} r={r}")
    # the step is consumed: the next synchronisation is a plain one
    fill_from_host(grads, init)
    for r in range(R):
        for v in range(P):
            og[r][v][...] = init[r][v]
    order = WG.permutation(70 + case, P)
    red.sync(order)
    orc.sync(order)
    got = snapshot(grads)
    for v in range(P):
        for r in range(R):
            assert_bits_equal(got[v][r], og[r][v], f"{name} next sync v={v} r={r}")
    red.close()
