"""The allocation-free binding (ddpb_bind_static) against ddpb_bind and the
oracle: the same bits, 0 ULP, every element of every replica, on two calls in
a row (the second with a smaller model that takes the static array over), in
fused and staged modes; a model too large for the array is refused."""
import pytest
import torch

import ddp_bucketed_gradient_amd as D
from gpu_util import require_gpu, say, alloc_grads, fill_from_host, snapshot, assert_bits_equal
from oracle import reducer as OR
from workloads import gen as WG

pytestmark = pytest.mark.gpu

# first call: several buckets, ragged tails, segments spanning 8192 elements
BIG = ([1, 3, 4097, 8193, 12345, 64, 20000, 5, 70000, 2, 777, 4096, 0, 16384, 33000], 8, 4 * 20000)
# second call: a smaller model and replica count
SMALL = ([10, 100, 4099, 7, 513], 3, 4 * 2000)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _case(numels, R, cap, seed):
    host = [[WG.normal(WG.seed_of(11, r, v, seed), n).numpy() for v, n in enumerate(numels)] for r in range(R)]
    order = WG.permutation(seed, len(numels))
    orc = OR.Reducer(numels, R, cap)
    og = [[h.copy() for h in row] for row in host]
    orc.bind(og)
    orc.sync(order)
    return host, order, og, orc.launch_log


@pytest.mark.parametrize("mode", [D.MODE_FUSED, D.MODE_STAGED])
def test_static_binding_matches_bind_twice(mode):
    previous = None
    for call, (numels, R, cap) in enumerate([BIG, SMALL]):
        say(f"bind_static call {call}: mode={mode} P={len(numels)} R={R}")
        host, order, want, want_log = _case(numels, R, cap, 20 + 2 * call + mode)
        ref = D.Reducer([(n,) for n in numels], R, cap)
        g_ref = alloc_grads(numels, R)
        ref.bind(g_ref, mode=mode)
        fill_from_host(g_ref, host)
        ref.sync(order)
        st = D.Reducer([(n,) for n in numels], R, cap)
        g_st = alloc_grads(numels, R)
        st.bind_static(g_st, mode=mode)
        if previous is not None:             # the array now holds this handle's tables
            with pytest.raises(D.DdpbError) as e:
                previous.sync()
            assert e.value.code == D.E_STATE
            previous.reset()
        fill_from_host(g_st, host)
        st.sync(order)
        got_ref, got_st = snapshot(g_ref), snapshot(g_st)
        assert st.launch_log() == ref.launch_log() == want_log
        for v in range(len(numels)):
            for r in range(R):
                assert_bits_equal(got_st[v][r], got_ref[v][r], f"call={call} static vs bind v={v} r={r}")
                assert_bits_equal(got_st[v][r], want[r][v], f"call={call} static vs oracle v={v} r={r}")
        # a second sync on the same static binding, fresh inputs
        host2, _, want2, _ = _case(numels, R, cap, 40 + call + mode)
        fill_from_host(g_st, host2)
        st.sync(order)
        got2 = snapshot(g_st)
        orc = OR.Reducer(numels, R, cap)
        og = [[h.copy() for h in row] for row in host2]
        orc.bind(og)
        orc.sync(order)
        for v in range(len(numels)):
            for r in range(R):
                assert_bits_equal(got2[v][r], og[r][v], f"call={call} second sync v={v} r={r}")
        ref.close()
        if previous is not None:
            previous.close()
        previous = st
    previous.close()


def test_static_binding_refuses_a_model_beyond_the_array():
    numels, R = [10_000_000], 8                 # staged: 9 flat copies of 40 MB
    red = D.Reducer([(n,) for n in numels], R, 0)
    grads = alloc_grads(numels, R)
    with pytest.raises(D.DdpbError) as e:
        red.bind_static(grads, mode=D.MODE_STAGED)
    assert e.value.code == D.E_ARG and "static array holds" in str(e.value)
    red.bind_static(grads, mode=D.MODE_FUSED)    # the tables alone fit
    host = [[WG.normal(WG.seed_of(12, r, 0), numels[0]).numpy()] for r in range(R)]
    fill_from_host(grads, host)
    red.sync()
    got = snapshot(grads)
    want = OR.fixed_order_mean([host[r][0] for r in range(R)])
    for r in range(R):
        assert_bits_equal(got[0][r], want, f"r={r}")
    red.close()


def test_static_binding_sync_captured_and_replayed():
    """A sync on a static binding recorded into a HIP graph and replayed three
    times with eager work between the replays: every replay leaves the
    oracle's bits (the inputs are refilled before each replay)."""
    numels, R, cap = SMALL[0] + [9000], 4, 4 * 3000
    red = D.Reducer([(n,) for n in numels], R, cap)
    grads = alloc_grads(numels, R)
    compute = torch.cuda.Stream()
    with torch.cuda.stream(compute):
        red.bind_static(grads, compute_stream=compute)
        host, order, want, _ = _case(numels, R, cap, 60)
        fill_from_host(grads, host)
        red.sync(order)                        # eager sync first: same bits
    got = snapshot(grads)
    for v in range(len(numels)):
        for r in range(R):
            assert_bits_equal(got[v][r], want[r][v], f"eager v={v} r={r}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=compute):
        red.sync(order)
    for rep in range(3):
        host, _, _, _ = _case(numels, R, cap, 61 + rep)
        orc = OR.Reducer(numels, R, cap)
        og = [[h.copy() for h in row] for row in host]
        orc.bind(og)
        orc.sync(order)
        with torch.cuda.stream(compute):
            fill_from_host(grads, host)
            torch.cuda.synchronize()
            g.replay()
        torch.cuda.synchronize()
        got = snapshot(grads)
        for v in range(len(numels)):
            for r in range(R):
                assert_bits_equal(got[v][r], og[r][v], f"replay {rep} v={v} r={r}")
    red.close()


def test_static_rebind_of_the_same_handle_on_another_stream():
    """A static binding re-bound by the same handle onto another compute stream
    while its last sync may still run: the rebind drains the device before it
    rewrites the array, so both syncs leave the oracle's bits."""
    numels, R, cap = BIG[0], 8, BIG[2]
    red = D.Reducer([(n,) for n in numels], R, cap)
    ga, gb = alloc_grads(numels, R), alloc_grads(numels, R)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    host_a, order, want_a, _ = _case(numels, R, cap, 70)
    host_b, _, _, _ = _case(numels, R, cap, 71)
    fill_from_host(ga, host_a)
    fill_from_host(gb, host_b)
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        red.bind_static(ga, compute_stream=sa)
        red.sync(order)                        # not waited for before the rebind
    with torch.cuda.stream(sb):
        red.bind_static(gb, compute_stream=sb)
        red.sync(order)
    torch.cuda.synchronize()
    orc = OR.Reducer(numels, R, cap)
    og = [[h.copy() for h in row] for row in host_b]
    orc.bind(og)
    orc.sync(order)
    got_a, got_b = snapshot(ga), snapshot(gb)
    for v in range(len(numels)):
        for r in range(R):
            assert_bits_equal(got_a[v][r], want_a[r][v], f"first binding v={v} r={r}")
            assert_bits_equal(got_b[v][r], og[r][v], f"second binding v={v} r={r}")
    red.close()
