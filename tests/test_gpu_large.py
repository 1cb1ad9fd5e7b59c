"""GPU parity for one tensor larger than 2^31 elements (8.6 GB per replica):
every element offset inside the kernels and the plan is 64-bit, so a segment
that starts past 2^31 must read and write exactly the elements the oracle
averages. Windows at the start, across the 2^31 boundary and at the end, plus
seeded scattered positions, are compared with the oracle bit for bit; every
element is compared across replicas (they must all hold the same mean).

The small variables around the large one put it at bucket offset 7 (cap
25 MiB: the staged pack and copy-back take their 4-byte path) or alone in its
bucket (cap 0)."""
import gc

import numpy as np
import pytest
import torch

import ddp_bucketed_gradient_amd as D
from gpu_util import require_gpu, say, assert_bits_equal
from oracle import reducer as OR
from workloads import gen as WG

pytestmark = pytest.mark.gpu
MiB = 1 << 20
BIG = (1 << 31) + 9221            # a full segment at 2^31, then a ragged one
NUMELS = [5, BIG, 7]
R = 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()


def _windows():
    """(start, length) windows of the large tensor, then scattered positions."""
    edge = 1 << 31
    wins = [(0, 20000), (edge - 16391, 16391 + 4096), (BIG - 20000, 20000)]
    rng = np.random.default_rng(31)
    pos = np.unique(rng.integers(0, BIG, size=256))
    wins += [(int(p), 1) for p in pos]
    return wins


def _take(t, wins):
    """Host float32 copies of the windows of one device tensor."""
    return [t[s:s + n].cpu().numpy().copy() for s, n in wins]


def _fill(grads, t=0):
    for r in range(R):
        for v, n in enumerate(NUMELS):
            WG.normal(WG.seed_of(12, r, v, t), n, "cuda", out=grads[r][v])


def _check(grads, before_small, before_big, wins, what):
    """The oracle on the small variables and on the large one's windows."""
    torch.cuda.synchronize()
    for v in (0, 2):
        want = OR.fixed_order_mean(before_small[v])
        for r in range(R):
            assert_bits_equal(grads[r][v].cpu().numpy(), want, f"{what} v={v} r={r}")
    for k, (s, n) in enumerate(wins):
        want = OR.fixed_order_mean([before_big[r][k] for r in range(R)])
        for r in range(R):
            assert_bits_equal(grads[r][1][s:s + n].cpu().numpy(), want, f"{what} window {k} at {s} r={r}")
    for r in range(1, R):
        assert torch.equal(grads[r][1], grads[0][1]), f"{what}: replicas differ"


@pytest.mark.parametrize("mode,cap_mib", [("fused", 25), ("fused", 0), ("staged", 25), ("view", 25)])
def test_tensor_beyond_int32_elements(mode, cap_mib):
    say(f"large tensor: numel={BIG} R={R} mode={mode} cap={cap_mib} MiB")
    wins = _windows()
    red = D.Reducer([(n,) for n in NUMELS], R, cap_mib * MiB)
    if mode == "view":
        grads = [[g.view(-1) for g in row] for row in red.bind_bucket_views()]
    else:
        grads = [[torch.empty(n, dtype=torch.float32, device="cuda") for n in NUMELS] for _ in range(R)]
        red.bind(grads, mode=D.MODE_STAGED if mode == "staged" else D.MODE_FUSED)
    _fill(grads)
    torch.cuda.synchronize()
    before_small = {v: [grads[r][v].cpu().numpy().copy() for r in range(R)] for v in (0, 2)}
    before_big = [_take(grads[r][1], wins) for r in range(R)]
    red.sync()
    _check(grads, before_small, before_big, wins, f"{mode} cap={cap_mib}")
    red.close()
    del grads, red
    gc.collect()
    torch.cuda.empty_cache()


def test_no_sync_accumulate_beyond_int32_elements():
    """Two bf16 micro-steps accumulated into the fp32 gradients, then one
    synchronisation; the oracle runs the same steps on the windows (the
    arithmetic is elementwise, so each window is a variable of its own)."""
    say(f"large tensor no_sync: numel={BIG} R={R}")
    wins = _windows()
    red = D.Reducer([(n,) for n in NUMELS], R, 25 * MiB)
    grads = [[torch.empty(n, dtype=torch.float32, device="cuda") for n in NUMELS] for _ in range(R)]
    red.bind(grads)
    parts = [(v, 0, NUMELS[v]) for v in (0, 2)] + [(1, s, n) for s, n in wins]
    orc = OR.Reducer([n for _, _, n in parts], R, 1 << 62)
    og = [[np.zeros(n, np.float32) for _, _, n in parts] for _ in range(R)]
    orc.bind(og)
    for t in range(2):
        steps = [[WG.normal_bf16(WG.seed_of(12, r, v, 10 + t), n, "cuda") for v, n in enumerate(NUMELS)]
                 for r in range(R)]
        host = [[steps[r][v][s:s + n].view(torch.int16).cpu().numpy().view(np.uint16).copy()
                 for v, s, n in parts] for r in range(R)]
        red.no_sync_accumulate(steps, first_step=(t == 0))
        orc.no_sync_accumulate(host, first=(t == 0))
        torch.cuda.synchronize()
        del steps
        torch.cuda.empty_cache()
    red.sync()
    orc.sync()
    torch.cuda.synchronize()
    for k, (v, s, n) in enumerate(parts):
        for r in range(R):
            assert_bits_equal(grads[r][v][s:s + n].cpu().numpy(), og[r][k], f"no_sync part {k} (v={v} at {s}) r={r}")
    for v in range(len(NUMELS)):
        assert torch.equal(grads[1][v], grads[0][v]), f"no_sync: replicas differ at v={v}"
    red.close()
    del grads, red
    gc.collect()
    torch.cuda.empty_cache()
