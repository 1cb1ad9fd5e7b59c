"""GPU parity: the HIP path, called through the C ABI, against the oracle,
bit for bit (0 ULP) on the same seeded inputs.

Small cases span several segments and ragged tails and run the whole oracle;
ResNet-50 shapes run at full size here, every element. The other full-size
workloads (BERT-large with the cap sweep, bucket views and used flags, BERT-base
no_sync, the overlapped MLP backward) are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import ddp_bucketed_gradient_amd as D
from gpu_util import require_gpu, say, alloc_grads, fill_from_host, snapshot, assert_bits_equal
from oracle import reducer as OR
from oracle import linear10 as OL
from workloads import gen as WG, configs as WC

pytestmark = pytest.mark.gpu
MiB = 1 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _oracle_sync(numels, R, cap, host, order):
    red = OR.Reducer(numels, R, cap)
    g = [[np.array(host[r][v], np.float32, copy=True) for v in range(len(numels))] for r in range(R)]
    red.bind(g)
    red.sync(order)
    return g, red.launch_log


def _host_inputs(seed, numels, R, kind="normal"):
    if kind == "dyadic":
        return [[WG.dyadic(seed * 7919 + r * 131 + v, n) for v, n in enumerate(numels)] for r in range(R)]
    return [[WG.normal(WG.seed_of(9, r, v, seed % 100), n).numpy() for v, n in enumerate(numels)]
            for r in range(R)]


RAGGED = [1, 3, 4, 5, 63, 64, 65, 255, 1000, 4095, 4096, 4097, 8191, 8193, 12345, 20000, 2, 777]


@pytest.mark.parametrize("R", [1, 2, 3, 5, 8, 16, 17, 20, 24, 33, 64])
@pytest.mark.parametrize("mode", [D.MODE_FUSED, D.MODE_STAGED])
def test_ragged_parity(R, mode):
    numels = RAGGED
    cap = 4 * 9000
    order = WG.permutation(R * 10 + mode, len(numels))
    say(f"ragged R={R} mode={mode} P={len(numels)} cap={cap}")
    red = D.Reducer([(n,) for n in numels], R, cap)
    grads = alloc_grads(numels, R)
    red.bind(grads, mode=mode)
    for it in range(2):
        host = _host_inputs(it + R, numels, R, "dyadic" if (it == 1 and R == 3) else "normal")
        fill_from_host(grads, host)
        red.sync(order)
        got = snapshot(grads)
        want, log = _oracle_sync(numels, R, cap, host, order)
        assert red.launch_log() == log
        for v in range(len(numels)):
            for r in range(R):
                assert_bits_equal(got[v][r], want[r][v], f"it={it} v={v} r={r}")
    red.close()


@pytest.mark.parametrize("n_side", [2, 3])
def test_multiple_side_streams(n_side):
    numels = RAGGED * 2
    R = 4
    red = D.Reducer([(n,) for n in numels], R, 0)            # one bucket per tensor
    grads = alloc_grads(numels, R)
    sides = [torch.cuda.Stream() for _ in range(n_side)]
    red.bind(grads, side_streams=sides)
    host = _host_inputs(3, numels, R)
    fill_from_host(grads, host)
    order = list(range(len(numels) - 1, -1, -1))
    red.sync(order)
    got = snapshot(grads)
    want, _ = _oracle_sync(numels, R, 0, host, order)
    for v in range(len(numels)):
        for r in range(R):
            assert_bits_equal(got[v][r], want[r][v], f"v={v} r={r}")


def test_special_values():
    vals = np.array([0.0, -0.0, 1e-45, -1e-45, 2e-45, 1.1754942e-38, 3.4e38, 3.4e38, -3.4e38,
                     np.inf, -np.inf, np.nan, 1.0, 2.0 ** 24, 1.0, -(2.0 ** 24)], dtype=np.float32)
    for RR in (2, 3, 8):
        host = [[np.roll(vals, r * 3 + 1).copy()] for r in range(RR)]
        for mode in (D.MODE_FUSED, D.MODE_STAGED):
            red = D.Reducer([(vals.size,)], RR, 0)
            grads = alloc_grads([vals.size], RR)
            red.bind(grads, mode=mode)
            fill_from_host(grads, host)
            red.sync()
            got = snapshot(grads)
            with np.errstate(invalid="ignore", over="ignore"):   # Inf - Inf and overflow are the point
                want, _ = _oracle_sync([vals.size], RR, 0, host, [0])
            for r in range(RR):
                assert_bits_equal(got[0][r], want[r][0], f"R={RR} mode={mode}")
    # subnormal results must not be flushed: (2^-149 + 2^-149) / 2
    red = D.Reducer([(8,)], 2, 0)
    grads = alloc_grads([8], 2)
    red.bind(grads)
    tiny = np.full(8, np.float32(2.0 ** -149), np.float32)
    fill_from_host(grads, [[tiny], [tiny]])
    red.sync()
    assert np.array_equal(snapshot(grads)[0][0].view(np.uint32), np.ones(8, np.uint32))


@pytest.mark.parametrize("R", [4, 20, 24])
def test_unaligned_views_take_the_scalar_path(R):
    numels = [5, 4096, 37, 1000]
    base = [torch.zeros(sum(numels) + 16, device="cuda") for _ in range(R)]
    grads = []
    for r in range(R):
        off, row = 1, []                     # 4-byte offset: not 16-byte aligned
        for n in numels:
            row.append(base[r][off:off + n])
            off += n
        grads.append(row)
    host = _host_inputs(11, numels, R)
    fill_from_host(grads, host)
    for mode in (D.MODE_FUSED, D.MODE_STAGED):
        fill_from_host(grads, host)
        red = D.Reducer([(n,) for n in numels], R, 4 * 2000)
        red.bind(grads, mode=mode)
        red.sync()
        got = snapshot(grads)
        want, _ = _oracle_sync(numels, R, 4 * 2000, host, list(range(len(numels) - 1, -1, -1)))
        for v in range(len(numels)):
            for r in range(R):
                assert_bits_equal(got[v][r], want[r][v], f"mode={mode} v={v} r={r}")
        red.close()


def test_empty_tensors_and_empty_model():
    numels = [0, 7, 0, 4100, 0]
    R = 2
    red = D.Reducer([(n,) for n in numels], R, 0)
    grads = alloc_grads(numels, R)
    red.bind(grads)
    host = _host_inputs(2, numels, R)
    fill_from_host(grads, host)
    red.sync()
    got = snapshot(grads)
    want, _ = _oracle_sync(numels, R, 0, host, list(range(4, -1, -1)))
    for v in (1, 3):
        for r in range(R):
            assert_bits_equal(got[v][r], want[r][v])
    empty = D.Reducer([], 4)
    empty.bind([[] for _ in range(4)])
    empty.sync()


def test_linear10_example():
    """nn.Linear(10, 10), two ranks, loss mean(out^2), lr 0.001: after the
    step every replica holds the same parameters."""
    R = 2
    W0, b0 = WG.linear10_init(0)                          # broadcast: every rank takes rank 0's
    params = [[W0.clone().cuda().requires_grad_(), b0.clone().cuda().requires_grad_()] for _ in range(R)]
    for r in range(R):
        x = WG.linear10_batch(r).cuda()
        out = x @ params[r][0].T + params[r][1]
        out.square().mean().backward()
    grads = [[p[0].grad, p[1].grad] for p in params]
    red = D.Reducer([(10, 10), (10,)], R)
    assert red.buckets() == [[1, 0]]
    red.bind(grads)
    local = snapshot(grads)
    red.sync()
    got = snapshot(grads)
    host = [[local[v][r].reshape(-1) for v in range(2)] for r in range(R)]
    want, _ = _oracle_sync([100, 10], R, 25 * MiB, host, [1, 0])
    for v in range(2):
        for r in range(R):
            assert_bits_equal(got[v][r].reshape(-1), want[r][v], f"v={v} r={r}")
    # the averaged gradient agrees with the float64 closed form to fp32 accuracy
    cf = [OL.grads(WG.linear10_batch(r).numpy(), W0.numpy(), b0.numpy()) for r in range(R)]
    mean_dW = (cf[0][0].astype(np.float64) + cf[1][0]) / 2
    assert np.allclose(got[0][0], mean_dW, rtol=1e-5, atol=1e-7)
    with torch.no_grad():
        for r in range(R):
            for p in params[r]:
                p.add_(p.grad, alpha=-0.001)
    for r in range(1, R):
        for p, q in zip(params[r], params[0]):
            assert torch.equal(p, q)


def test_stream_ordering_with_delayed_producer():
    """The last gradient is written on the compute stream behind a long chain
    of GEMMs; the reduction on the side stream must wait for it."""
    numels = [4096 * 3 + 5, 999, 50000]
    R = 4
    red = D.Reducer([(n,) for n in numels], R, 0)
    grads = alloc_grads(numels, R)
    for row in grads:
        for g in row:
            g.zero_()
    red.bind(grads)
    host = _host_inputs(21, numels, R)
    staged = [[torch.from_numpy(h).cuda() for h in row] for row in host]
    torch.cuda.synchronize()
    a = torch.randn(2048, 2048, device="cuda")
    for v in (2, 1, 0):                       # reverse index = bucket order
        for _ in range(40):
            a = torch.tanh(a @ a * 1e-3)       # delay on the compute stream
        for r in range(R):
            grads[r][v].copy_(staged[r][v])
        red.mark_ready(v)                     # host does not wait
    red.finalize()
    got = snapshot(grads)
    want, _ = _oracle_sync(numels, R, 0, host, [2, 1, 0])
    for v in range(3):
        for r in range(R):
            assert_bits_equal(got[v][r], want[r][v], f"v={v} r={r}")


def _delay(stream, n=40):
    """Queue about 40 dependent fp32 GEMMs (milliseconds of work) on `stream`."""
    with torch.cuda.stream(stream):
        a = torch.randn(2048, 2048, device="cuda")
        for _ in range(n):
            a = torch.tanh(a @ a * 1e-3)
    return a


@pytest.mark.parametrize("n_side", [1, 2, 3])
@pytest.mark.parametrize("timed", [False, True])
@pytest.mark.parametrize("kind", ["fused", "staged", "sync_step"])
def test_finalize_orders_later_compute_work(kind, timed, n_side):
    """Work queued on the compute stream after finalize sees the averaged
    gradients without any host synchronisation ([Li] 3.2: the reduction is
    done when backward returns). Each side stream is held back by a GEMM chain
    before the sync, so the device copies queued on the compute stream right
    after finalize would read unreduced gradients if the join did not order
    them. Two iterations (the join's events are per iteration); with three
    side streams and two buckets one stream stays unused."""
    numels = [4096 * 3 + 5, 999, 50000, 70001, 7]
    R, P = 4, len(numels)
    cap = 4 * 60000 if n_side == 3 else 0         # 2 buckets, or one per tensor
    say(f"join order kind={kind} timed={timed} n_side={n_side}")
    compute = torch.cuda.Stream()
    sides = [torch.cuda.Stream() for _ in range(n_side)]
    red = D.Reducer([(n,) for n in numels], R, cap)
    grads = alloc_grads(numels, R)
    mode = D.MODE_STAGED if kind == "staged" else D.MODE_FUSED
    red.bind(grads, compute_stream=compute, side_streams=sides, mode=mode,
             flags=D.BIND_TIME_LAUNCHES if timed else 0)
    order = list(range(P - 1, -1, -1))
    for it in range(2):
        host = _host_inputs(41 + it, numels, R)
        steps_host = _host_inputs(51 + it, numels, R) if kind == "sync_step" else None
        fill_from_host(grads, host)
        steps = [[torch.from_numpy(h).cuda() for h in row] for row in steps_host] if steps_host else None
        torch.cuda.synchronize()
        keep = [_delay(s) for s in sides]
        with torch.cuda.stream(compute):
            if steps is not None:
                red.set_sync_step(steps)
            for v in order:
                red.mark_ready(v)
            red.finalize()
            copies = [[g.clone() for g in row] for row in grads]   # queued behind the join only
        torch.cuda.synchronize()
        del keep
        ref = OR.Reducer(numels, R, cap)
        want = [[np.array(host[r][v], np.float32, copy=True) for v in range(P)] for r in range(R)]
        ref.bind(want)
        if steps_host is not None:
            ref.no_sync_accumulate(steps_host, first=False)
        ref.sync(order)
        assert red.launch_log() == ref.launch_log
        for r in range(R):
            for v in range(P):
                assert_bits_equal(copies[r][v].cpu().numpy(), want[r][v], f"it={it} r={r} v={v}")
    red.close()


def test_single_bucket_reduces_on_the_compute_stream():
    """A plan of one bucket reduces on the compute stream whatever side
    streams are bound: with both side streams held back by GEMM chains, the
    synchronised gradients are on the compute stream (and bit-exact) while the
    side streams are still busy, so nothing waited for them."""
    numels = [4096 * 3 + 5, 999, 7]
    R, P = 4, len(numels)
    compute = torch.cuda.Stream()
    sides = [torch.cuda.Stream() for _ in range(2)]
    red = D.Reducer([(n,) for n in numels], R, 1 << 30)
    assert red.num_buckets == 1
    grads = alloc_grads(numels, R)
    red.bind(grads, compute_stream=compute, side_streams=sides)
    host = _host_inputs(61, numels, R)
    fill_from_host(grads, host)
    torch.cuda.synchronize()
    keep = [_delay(s, 200) for s in sides]
    with torch.cuda.stream(compute):
        red.sync(list(range(P - 1, -1, -1)))
        copies = [[g.clone() for g in row] for row in grads]
        done = torch.cuda.Event()
        done.record(compute)
    done.synchronize()
    busy = [not s.query() for s in sides]
    torch.cuda.synchronize()
    del keep
    assert all(busy), "the single bucket waited for the side streams"
    want, log = _oracle_sync(numels, R, 1 << 30, host, list(range(P - 1, -1, -1)))
    assert red.launch_log() == log
    for r in range(R):
        for v in range(P):
            assert_bits_equal(copies[r][v].cpu().numpy(), want[r][v], f"r={r} v={v}")
    red.close()


@pytest.mark.parametrize("layout", ["compute_only", "compute_and_side"])
def test_compute_stream_as_side_stream(layout):
    """Buckets bound to the compute stream itself run without cross-stream
    events; mixed with a separate side stream, that stream's buckets still wait
    for a producer delayed on the compute stream, and finalize still joins it."""
    numels = [4096 * 3 + 5, 999, 50000, 7]
    R = 4
    P = len(numels)
    say(f"compute stream as side stream: {layout}")
    red = D.Reducer([(n,) for n in numels], R, 0)
    grads = alloc_grads(numels, R)
    compute = torch.cuda.current_stream()
    sides = [compute] if layout == "compute_only" else [compute, torch.cuda.Stream()]
    red.bind(grads, compute_stream=compute, side_streams=sides, flags=D.BIND_TIME_LAUNCHES)
    for it in range(2):
        host = _host_inputs(31 + it, numels, R)
        staged = [[torch.from_numpy(h).cuda() for h in row] for row in host]
        torch.cuda.synchronize()
        a = torch.randn(2048, 2048, device="cuda")
        for v in range(P - 1, -1, -1):             # reverse index = bucket order
            for _ in range(30):
                a = torch.tanh(a @ a * 1e-3)       # delay on the compute stream
            for r in range(R):
                grads[r][v].copy_(staged[r][v])
            red.mark_ready(v)                     # host does not wait
        red.finalize()
        got = snapshot(grads)
        want, _ = _oracle_sync(numels, R, 0, host, list(range(P - 1, -1, -1)))
        for v in range(P):
            for r in range(R):
                assert_bits_equal(got[v][r], want[r][v], f"{layout} it={it} v={v} r={r}")
        assert len(red.launch_times_ms()) == P
    red.close()


def test_parked_buckets_and_device_stamps():
    numels = [3000] * 12
    R = 2
    red = D.Reducer([(n,) for n in numels], R, 0)
    grads = alloc_grads(numels, R)
    red.bind(grads, flags=D.BIND_DEVICE_TIMESTAMPS | D.BIND_TIME_LAUNCHES)
    host = _host_inputs(4, numels, R)
    fill_from_host(grads, host)
    order = [11, 9, 8, 10, 7, 3, 4, 5, 6, 2, 0, 1]     # buckets 0, park, ..., so launches batch up
    red.sync(order)
    torch.cuda.synchronize()
    got = snapshot(grads)
    want, log = _oracle_sync(numels, R, 0, host, order)
    rows, t0, t1 = red.launch_log(with_stamps=True)
    assert rows == log
    assert [b for b, _ in rows] == list(range(12))
    assert all(b > a for a, b in zip(t0, t0[1:]))           # one side stream: in order on the device
    assert all(e >= s for s, e in zip(t0, t1))
    assert all(s >= e for s, e in zip(t0[1:], t1))           # and never overlapping
    ms = red.launch_times_ms()
    assert len(ms) == 12 and all(m > 0 for m in ms)
    assert red.device_clock_hz() > 0
    for v in range(12):
        for r in range(R):
            assert_bits_equal(got[v][r], want[r][v])


def test_incomplete_iteration_then_recovery():
    numels = [100, 200, 300]
    R = 2
    red = D.Reducer([(n,) for n in numels], R, 0)
    grads = alloc_grads(numels, R)
    red.bind(grads)
    host = _host_inputs(8, numels, R)
    fill_from_host(grads, host)
    red.mark_ready(2)
    red.mark_ready(1)                 # variable 0 never gets its hook
    with pytest.raises(D.DdpbError) as e:
        red.finalize()
    assert e.value.code == -4
    with pytest.raises(D.DdpbError):
        red.ensure_prior_reduction_finished()
    torch.cuda.synchronize()
    red.reset()
    fill_from_host(grads, host)
    red.sync()
    got = snapshot(grads)
    want, _ = _oracle_sync(numels, R, 0, host, [2, 1, 0])
    for v in range(3):
        for r in range(R):
            assert_bits_equal(got[v][r], want[r][v])


# --- no_sync -------------------------------------------------------------------

def _oracle_nosync_one(host_steps_v, R, k):
    """Oracle on a one-variable model: accumulate k micro-steps, then sync."""
    n = host_steps_v[0][0].size
    red = OR.Reducer([n], R, 0)
    g = [[np.zeros(n, np.float32)] for _ in range(R)]
    red.bind(g)
    for t in range(k):
        red.no_sync_accumulate([[host_steps_v[t][r]] for r in range(R)], first=(t == 0))
    red.sync()
    return [g[r][0] for r in range(R)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_no_sync_small(dtype):
    numels = RAGGED
    R, k = 4, 3
    red = D.Reducer([(n,) for n in numels], R, 4 * 10000)
    grads = alloc_grads(numels, R)
    red.bind(grads)
    steps = [[[WG.normal(WG.seed_of(4, r, v, t), n, "cuda").to(dtype) for v, n in enumerate(numels)]
              for r in range(R)] for t in range(k)]
    red.set_sync(False)
    for t in range(k - 1):
        red.no_sync_accumulate(steps[t], first_step=(t == 0))
        red.sync()                                         # hooks are no-ops
        assert red.launch_log() == [] or t > 0
    red.set_sync(True)
    red.no_sync_accumulate(steps[k - 1], first_step=(k == 1))
    red.sync()
    torch.cuda.synchronize()
    for v, n in enumerate(numels):
        if dtype == torch.bfloat16:
            hs = [[steps[t][r][v].view(torch.int16).cpu().numpy().view(np.uint16) for r in range(R)] for t in range(k)]
        else:
            hs = [[steps[t][r][v].cpu().numpy() for r in range(R)] for t in range(k)]
        want = _oracle_nosync_one(hs, R, k)
        for r in range(R):
            assert_bits_equal(grads[r][v].cpu().numpy(), want[r], f"v={v} r={r}")


# --- full-size workloads -----------------------------------------------------------

def _device_inputs(cfg, grads, t=0):
    for r, row in enumerate(grads):
        for v, g in enumerate(row):
            WG.normal(WG.seed_of(cfg, r, v, t), g.numel(), "cuda", out=g)


def test_config2_resnet50_full():
    w = WC.RESNET50
    numels = w.numels()
    say(f"{w.name}: P={len(numels)} R={w.R}")
    red = D.Reducer([p.shape for p in w.params()], w.R, w.cap_bytes)
    assert red.num_buckets == 4
    grads = alloc_grads(numels, w.R)
    red.bind(grads)
    _device_inputs(w.cfg, grads)
    host_in = snapshot(grads)
    red.sync(w.ready_order())
    got = snapshot(grads)
    host = [[host_in[v][r] for v in range(len(numels))] for r in range(w.R)]
    want, log = _oracle_sync(numels, w.R, w.cap_bytes, host, w.ready_order())
    assert red.launch_log() == log
    for v in range(len(numels)):
        for r in range(w.R):
            assert_bits_equal(got[v][r], want[r][v], f"v={v} r={r}")


@pytest.mark.parametrize("mode", [D.MODE_FUSED, D.MODE_STAGED])
@pytest.mark.parametrize("blocks", [1, 3])
def test_capped_grid_parity(mode, blocks):
    """With the workgroups of each launch capped, every wavefront strides over
    several segments; the result must not change."""
    numels = RAGGED + [70000, 3, 131072]
    R = 8
    order = WG.permutation(77, len(numels))
    red = D.Reducer([(n,) for n in numels], R, 4 * 30000)
    red.set_launch_blocks(blocks)
    grads = alloc_grads(numels, R)
    red.bind(grads, mode=mode)
    host = _host_inputs(40 + blocks, numels, R)
    fill_from_host(grads, host)
    red.sync(order)
    got = snapshot(grads)
    want, log = _oracle_sync(numels, R, 4 * 30000, host, order)
    assert red.launch_log() == log
    for v in range(len(numels)):
        for r in range(R):
            assert_bits_equal(got[v][r], want[r][v], f"blocks={blocks} v={v} r={r}")


@pytest.mark.parametrize("R", [8, 20, 24])
@pytest.mark.parametrize("wg", [0, 1, 2])
@pytest.mark.parametrize("flags", [False, True])
@pytest.mark.parametrize("mode", [D.MODE_FUSED, D.MODE_STAGED])
def test_workgroups_per_cu_parity(R, wg, flags, mode):
    """The LDS reservation that bounds reduction workgroups per CU, for the
    fused kernels with and without used flags, the generic-R kernel and the
    staged trio: same bits as the oracle, several buckets, two side streams."""
    numels = RAGGED + [70000, 3, 131072]
    say(f"workgroups_per_cu={wg} R={R} flags={flags} mode={mode}")
    red = D.Reducer([(n,) for n in numels], R, 4 * 30000)
    red.set_workgroups_per_cu(wg)
    grads = alloc_grads(numels, R)
    red.bind(grads, mode=mode)
    orc = OR.Reducer(numels, R, 4 * 30000)
    host = _host_inputs(60 + wg + 3 * R, numels, R)
    og = [[np.array(h, np.float32, copy=True) for h in row] for row in host]
    orc.bind(og)
    fill_from_host(grads, host)
    order = WG.permutation(78, len(numels))
    if flags:
        rng = np.random.default_rng(wg + R)
        used = rng.random((R, len(numels))) < 0.7
        red.set_local_used(used)
        orc.set_local_used(used)
        G = used.any(axis=0)
        order = [v for v in order if G[v]]
    red.sync(order)
    orc.sync(order)
    got = snapshot(grads)
    assert red.launch_log() == orc.launch_log
    for v in range(len(numels)):
        for r in range(R):
            assert_bits_equal(got[v][r], og[r][v], f"wg={wg} R={R} v={v} r={r}")
    red.close()


def test_two_handles_interleaved_on_shared_streams():
    """Two reducers (different shapes, replica counts, modes) bound at once,
    sharing the compute and side streams, hooks interleaved: each must match
    its own oracle, so no state is shared between handles."""
    compute = torch.cuda.Stream()
    sides = [torch.cuda.Stream(), torch.cuda.Stream()]
    specs = [(RAGGED, 3, 4 * 9000, D.MODE_FUSED), ([70000, 5, 8192, 131072, 1], 8, 4 * 40000, D.MODE_STAGED)]
    reds, grads, wants, orders = [], [], [], []
    for k, (numels, R, cap, mode) in enumerate(specs):
        say(f"handle {k}: P={len(numels)} R={R} mode={mode}")
        red = D.Reducer([(n,) for n in numels], R, cap)
        g = alloc_grads(numels, R)
        red.bind(g, compute_stream=compute, side_streams=sides, mode=mode)
        host = _host_inputs(90 + k, numels, R)
        fill_from_host(g, host)
        order = WG.permutation(91 + k, len(numels))
        want, _ = _oracle_sync(numels, R, cap, host, order)
        reds.append(red); grads.append(g); wants.append(want); orders.append(order)
    torch.cuda.synchronize()
    with torch.cuda.stream(compute):
        n = max(len(o) for o in orders)
        for i in range(n):                           # hooks of the two models interleaved
            for red, order in zip(reds, orders):
                if i < len(order):
                    red.mark_ready(order[i])
        for red in reds:
            red.finalize()
    for k, (numels, R, _, _) in enumerate(specs):
        got = snapshot(grads[k])
        for v in range(len(numels)):
            for r in range(R):
                assert_bits_equal(got[v][r], wants[k][r][v], f"handle {k} v={v} r={r}")
    for red in reds:
        red.close()


def test_step_table_reused_across_micro_steps():
    """One StepTable (checked and marshalled once) passed to several
    no_sync_accumulate calls and then as the synchronising step gives the same
    bits as the oracle fed the same steps each time."""
    numels = [5000, 3, 8192, 777]
    R, cap, k = 4, 4 * 6000, 3
    P = len(numels)
    say(f"step table reuse R={R} k={k}")
    red = D.Reducer([(n,) for n in numels], R, cap)
    grads = alloc_grads(numels, R)
    red.bind(grads)
    hs = [[WG.normal(WG.seed_of(13, r, v), n).to(torch.bfloat16) for v, n in enumerate(numels)] for r in range(R)]
    table = red.step_table([[h.cuda() for h in row] for row in hs])
    host_steps = [[h.view(torch.int16).numpy().view(np.uint16).copy() for h in row] for row in hs]
    orc = OR.Reducer(numels, R, cap)
    og = [[np.zeros(n, np.float32) for n in numels] for _ in range(R)]
    orc.bind(og)
    red.set_sync(False)
    orc.set_sync(False)
    for t in range(k - 1):
        red.no_sync_accumulate(table, first_step=(t == 0))
        orc.no_sync_accumulate(host_steps, first=(t == 0))
    red.set_sync(True)
    orc.set_sync(True)
    red.set_sync_step(table)
    orc.no_sync_accumulate(host_steps, first=False)
    order = WG.permutation(14, P)
    red.sync(order)
    orc.sync(order)
    got = snapshot(grads)
    for v in range(P):
        for r in range(R):
            assert_bits_equal(got[v][r], og[r][v], f"step table v={v} r={r}")
    red.close()


def test_roctx_ranges_leave_results_unchanged():
    """A binding with host-side roctx ranges (and launch timing) syncs, accumulates
    and runs a fused synchronising step with the oracle's bits."""
    numels = [4097, 10, 100, 8192, 3]
    R, cap = 4, 4 * 5000
    P = len(numels)
    say("roctx ranges")
    red = D.Reducer([(n,) for n in numels], R, cap)
    grads = alloc_grads(numels, R)
    red.bind(grads, flags=D.BIND_ROCTX | D.BIND_TIME_LAUNCHES)
    host = [[WG.normal(WG.seed_of(17, r, v), n).numpy() for v, n in enumerate(numels)] for r in range(R)]
    fill_from_host(grads, host)
    orc = OR.Reducer(numels, R, cap)
    og = [[h.copy() for h in row] for row in host]
    orc.bind(og)
    order = WG.permutation(18, P)
    red.sync(order)
    orc.sync(order)
    hs = [[WG.normal(WG.seed_of(19, r, v), n).numpy() for v, n in enumerate(numels)] for r in range(R)]
    ds = [[torch.from_numpy(h).cuda() for h in row] for row in hs]
    red.set_sync(False)
    orc.set_sync(False)
    red.no_sync_accumulate(ds, first_step=False)
    orc.no_sync_accumulate(hs, first=False)
    red.set_sync(True)
    orc.set_sync(True)
    red.set_sync_step(ds)
    orc.no_sync_accumulate(hs, first=False)
    red.sync(order)
    orc.sync(order)
    got = snapshot(grads)
    for v in range(P):
        for r in range(R):
            assert_bits_equal(got[v][r], og[r][v], f"roctx v={v} r={r}")
    red.close()


def test_wrong_size_step_is_refused_before_any_kernel():
    red = D.Reducer([(4,), (6,)], 2, 0)
    grads = alloc_grads([4, 6], 2)
    red.bind(grads)
    bad = [[torch.zeros(4, device="cuda"), torch.zeros(5, device="cuda")] for _ in range(2)]
    with pytest.raises(ValueError):
        red.no_sync_accumulate(bad, True)
    red.close()
