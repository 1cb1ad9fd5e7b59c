"""A bucketed synchronisation captured into a HIP graph: every replay, with
eager work and host synchronisation between replays, must give the oracle's
bits; the calls that cannot be captured are refused without breaking the
capture."""
import warnings

import pytest
import torch

import ddp_bucketed_gradient_amd as D
from gpu_util import require_gpu, say, fill_from_host, snapshot, assert_bits_equal
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
    return [[WG.normal(WG.seed_of(5, r, v, seed), n).numpy() for v, n in enumerate(NUMELS)] for r in range(R)]


def _oracle(host, R, cap, view, order):
    """The oracle's gradients after one sync of ``host`` (bucket views when
    ``view``: its gradients are views of its flat buckets)."""
    orc = OR.Reducer(NUMELS, R, cap, gradient_as_bucket_view=view)
    if view:
        og = orc.views()
        for r in range(R):
            for v in range(len(NUMELS)):
                og[r][v][...] = host[r][v]
    else:
        og = [[h.copy() for h in row] for row in host]
        orc.bind(og)
    orc.sync(order)
    return og


@pytest.mark.parametrize("mode", [D.MODE_FUSED, D.MODE_STAGED, "view"])
def test_captured_sync_replays_match_the_oracle(mode):
    R, cap = 4, 4 * 15000
    view = mode == "view"
    say(f"graph capture mode={mode}")
    order = WG.permutation(17, len(NUMELS))          # parked buckets included
    host = _host(1, R)
    compute = torch.cuda.Stream()
    sides = [torch.cuda.Stream(), torch.cuda.Stream()]
    red = D.Reducer([(n,) for n in NUMELS], R, cap)
    if view:
        grads = [[g.view(-1) for g in row] for row in red.bind_bucket_views(compute_stream=compute,
                                                                              side_streams=sides)]
        fill_from_host(grads, host)
    else:
        grads = [[torch.from_numpy(h).cuda() for h in row] for row in host]
        red.bind(grads, compute_stream=compute, side_streams=sides, mode=mode)
    og = _oracle(host, R, cap, view, order)
    torch.cuda.synchronize()
    with torch.cuda.stream(compute):
        red.sync(order)                              # one eager iteration first
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=compute):
        red.sync(order)
    torch.cuda.synchronize()
    for rep in range(3):
        fill_from_host(grads, host)                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(grads)
        for v in range(len(NUMELS)):
            for r in range(R):
                assert_bits_equal(got[v][r], og[r][v], f"replay {rep} v={v} r={r}")
    # eager iterations still work after capture and replays (fresh inputs)
    host2 = _host(2, R)
    fill_from_host(grads, host2)
    torch.cuda.synchronize()
    with torch.cuda.stream(compute):
        red.sync(order)
    got = snapshot(grads)
    og2 = _oracle(host2, R, cap, view, order)
    for v in range(len(NUMELS)):
        for r in range(R):
            assert_bits_equal(got[v][r], og2[r][v], f"eager after replays v={v} r={r}")
    del g
    red.close()


def test_uncapturable_calls_are_refused_inside_a_capture():
    R = 2
    grads = [[torch.zeros(n, device="cuda") for n in NUMELS] for _ in range(R)]
    steps = [[torch.zeros(n, device="cuda") for n in NUMELS] for _ in range(R)]
    compute = torch.cuda.Stream()
    red = D.Reducer([(n,) for n in NUMELS], R, 4 * 15000)
    red.bind(grads, compute_stream=compute, side_streams=[torch.cuda.Stream()])
    red.sync()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=compute):
        with pytest.raises(D.DdpbError) as e:
            red.no_sync_accumulate(steps, True)
        assert e.value.code == D.E_STATE
        with pytest.raises(D.DdpbError) as e:
            red.set_sync_step(steps, False)           # its table comes from host staging too
        assert e.value.code == D.E_STATE
        red.sync()                                   # the capture itself stays usable
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    timed = D.Reducer([(n,) for n in NUMELS], R, 0)   # one bucket per tensor
    timed.bind(grads, compute_stream=compute, side_streams=[torch.cuda.Stream()], flags=D.BIND_TIME_LAUNCHES)
    g2 = torch.cuda.CUDAGraph()
    with warnings.catch_warnings(), torch.cuda.graph(g2, stream=compute):
        warnings.simplefilter("ignore")              # torch notes that the graph is empty
        with pytest.raises(D.DdpbError) as e:
            timed.mark_ready(len(NUMELS) - 1)        # completes bucket 0: a timed launch
        assert e.value.code == D.E_STATE
    torch.cuda.synchronize()
    timed.reset()
    del g, g2
    red.close()
    timed.close()
