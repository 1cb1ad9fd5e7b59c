"""GPU parity at the workloads' full sizes, every element of every replica
against the oracle, 0 ULP, in the launch configuration the bench times (a
compute stream and two side streams from torch's pool, launch timing on).

Each replica's gradient of each variable is an own seeded draw, so after a
synchronisation the oracle's inputs are drawn again variable by variable on the
device (the same generator and seed give the same values; checked below) and
averaged on the host by the oracle. Config 5's replica-0 gradients come from a
bf16 backward; they are snapshotted on the compute stream right before each
hook (a device copy, no host synchronisation), so the reduction's wait on the
hook's ready event is what keeps it from reading a gradient the GEMM has not
written yet, and a wrong order shows up as a wrong mean.

Pages: [TP] "Distributed Data Parallel", "Internal Design" (every replica
ends with the average of all replicas' gradients); [Li] "Gradient Accumulation
(no_sync)"; [Li] "Overlapping Computation with Communication".
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import ddp_bucketed_gradient_amd as D
from gpu_util import (require_gpu, say, alloc_grads, assert_device_bits_equal, closed_form_launch_log,
                      host_workers, to_device_f32)
from oracle import plan as OP
from oracle import reducer as OR
from workloads import shapes as WS, gen as WG, configs as WC

# the oracle's host work at these sizes takes up to about a minute per test
pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _bench_streams():
    """The bench's streams: consecutive streams of torch's pool (distinct
    hardware queues), the compute stream current."""
    compute = torch.cuda.Stream()
    sides = [torch.cuda.Stream(), torch.cuda.Stream()]
    return compute, sides


CHUNK = 1 << 20


def _chunks(n, chunk=CHUNK):
    """Element ranges of at most `chunk`: the oracle's arrays and temporaries
    stay small enough for the host allocator to reuse (values are elementwise,
    so the oracle on a chunk gives that chunk's bits)."""
    return [(a, min(n, a + chunk)) for a in range(0, n, chunk)]


def _progress(i, n, what):
    if i % max(1, n // 4) == 0:
        say(f"  {what}: {i} of {n}")


class HostStage:
    """Host buffers, touched once and reused, that device tensors are copied
    back into (fresh host memory costs a page fault per 4 KiB)."""

    def __init__(self, count, max_elems, dtype=np.float32):
        self.bufs = [np.empty(max(max_elems, 1), dtype) for _ in range(count)]

    def fetch(self, i, dev):
        out = self.bufs[i][:dev.numel()]
        host = torch.from_numpy(out.view(np.int16) if out.dtype == np.uint16 else out)
        host.copy_(dev.reshape(-1).view(torch.int16) if dev.dtype == torch.bfloat16 else dev.reshape(-1))
        return out


def _regen_dev(cfg, r, v, n):
    return WG.normal(WG.seed_of(cfg, r, v), n, "cuda")


def _oracle_mean(pool, bufs, out):
    """The oracle's fixed-order mean of the replicas' buffers, chunk by chunk
    on the host threads, into out."""
    def job(ab):
        a, b = ab
        out[a:b] = OR.fixed_order_mean([x[a:b] for x in bufs])
    list(pool.map(job, _chunks(out.size)))
    return out


# --- config 3: BERT-large shapes, R = 8, the cap sweep ------------------------------

@pytest.fixture(scope="module")
def bert_large_means():
    """The oracle's fixed-order mean of every BERT-large variable over the 8
    replicas' seeded gradients (the values do not depend on the cap)."""
    w = WC.BERT_LARGE
    numels = w.numels()
    R = w.R
    say(f"oracle means for {w.name}: {len(numels)} variables, R={R}")
    # the draw into a preallocated tensor (as the workload fills gradients)
    # equals a fresh draw of the same seed
    for v in (0, 3, 390):
        a = torch.empty(numels[v], dtype=torch.float32, device="cuda")
        WG.normal(WG.seed_of(3, 5, v), numels[v], "cuda", out=a)
        assert torch.equal(a.view(torch.int32), _regen_dev(3, 5, v, numels[v]).view(torch.int32))
    stage = HostStage(R, max(numels))
    means = {}
    with ThreadPoolExecutor(host_workers()) as pool:
        for v, n in enumerate(numels):
            _progress(v, len(numels), "oracle means")
            bufs = [stage.fetch(r, _regen_dev(3, r, v, n)) for r in range(R)]
            means[v] = _oracle_mean(pool, bufs, np.empty(n, np.float32))
    say("oracle means ready")
    return means


def _fill(cfg, grads):
    for r, row in enumerate(grads):
        for v, g in enumerate(row):
            WG.normal(WG.seed_of(cfg, r, v), g.numel(), "cuda", out=g)


@pytest.fixture(scope="module")
def bert_large_grads():
    w = WC.BERT_LARGE
    return alloc_grads(w.numels(), w.R)


@pytest.mark.parametrize("cap_mib", WC.CAP_SWEEP_MIB)
def test_config3_bert_large_every_element(cap_mib, bert_large_means, bert_large_grads):
    w = WC.bert_large_cap(cap_mib)
    numels = w.numels()
    P, R = len(numels), w.R
    say(f"{w.name}: P={P} R={R} every element")
    compute, sides = _bench_streams()
    grads = bert_large_grads
    red = D.Reducer([p.shape for p in w.params()], R, w.cap_bytes)
    want_buckets = OP.compute_bucket_assignment_by_size(numels, 4, w.cap_bytes)
    assert red.buckets() == want_buckets
    with torch.cuda.stream(compute):
        red.bind(grads, compute_stream=compute, side_streams=sides, flags=D.BIND_TIME_LAUNCHES)
        _fill(3, grads)
        red.sync(w.ready_order())
    torch.cuda.synchronize()
    assert red.launch_log() == closed_form_launch_log(want_buckets, w.ready_order())
    for v in range(P):
        want = to_device_f32(bert_large_means[v])
        for r in range(R):
            assert_device_bits_equal(grads[r][v], want, f"cap={cap_mib} v={v} r={r}")
    red.close()


def test_config3_staged_every_element(bert_large_means, bert_large_grads):
    """The staged path (pack into flat buckets, mean, copy back) at full size,
    as the bench's --mode staged binds it (12 GB of caller workspace)."""
    w = WC.BERT_LARGE
    numels = w.numels()
    P, R = len(numels), w.R
    say(f"{w.name} staged every element")
    compute, sides = _bench_streams()
    grads = bert_large_grads
    red = D.Reducer([p.shape for p in w.params()], R, w.cap_bytes)
    with torch.cuda.stream(compute):
        red.bind(grads, compute_stream=compute, side_streams=sides, mode=D.MODE_STAGED,
                 flags=D.BIND_TIME_LAUNCHES)
        _fill(3, grads)
        red.sync(w.ready_order())
    torch.cuda.synchronize()
    assert red.launch_log() == closed_form_launch_log(red.buckets(), w.ready_order())
    for v in range(P):
        want = to_device_f32(bert_large_means[v])
        for r in range(R):
            assert_device_bits_equal(grads[r][v], want, f"staged v={v} r={r}")
    red.close()


@pytest.mark.parametrize("R", [20, 32])
def test_generic_replica_count_bert_large_every_element(R):
    """BERT-large shapes at R = 20 and 32 (the bench's --replicas), where the
    replica count is a run-time argument of the reduction kernel: every
    element of every replica against the oracle's fixed-order mean."""
    w = WC.BERT_LARGE
    numels = w.numels()
    P = len(numels)
    say(f"{w.name} at R={R} every element")
    compute, sides = _bench_streams()
    grads = alloc_grads(numels, R)
    red = D.Reducer([p.shape for p in w.params()], R, w.cap_bytes)
    with torch.cuda.stream(compute):
        red.bind(grads, compute_stream=compute, side_streams=sides, flags=D.BIND_TIME_LAUNCHES)
        _fill(3, grads)
        red.sync(w.ready_order())
    torch.cuda.synchronize()
    assert red.launch_log() == closed_form_launch_log(red.buckets(), w.ready_order())
    stage = HostStage(R, max(numels))
    out = np.empty(max(numels), np.float32)
    with ThreadPoolExecutor(host_workers()) as pool:
        for v, n in enumerate(numels):
            _progress(v, P, f"oracle at R={R}")
            bufs = [stage.fetch(r, _regen_dev(3, r, v, n)) for r in range(R)]
            want = to_device_f32(_oracle_mean(pool, bufs, out[:n]))
            for r in range(R):
                assert_device_bits_equal(grads[r][v], want, f"R={R} v={v} r={r}")
    red.close()
    del grads


@pytest.mark.parametrize("param_mib,cap_mib", [(4, 4), (4, 16), (4, 64), (1, 4), (1, 16), (1, 64)])
def test_blog_payload_every_element(param_mib, cap_mib):
    """The blog's 48 MiB payload per replica, R = 4, as 12 x 4 MiB or 48 x 1 MiB
    parameters under caps of 4, 16 and 64 MiB (the bench's --config 6)."""
    base = WC.BLOG_COARSE4 if param_mib == 4 else WC.BLOG_FINE1
    numels = base.numels()
    P, R, cap = len(numels), base.R, cap_mib * WS.MiB
    say(f"{base.name} cap {cap_mib} MiB every element")
    compute, sides = _bench_streams()
    grads = alloc_grads(numels, R)
    red = D.Reducer([p.shape for p in base.params()], R, cap)
    with torch.cuda.stream(compute):
        red.bind(grads, compute_stream=compute, side_streams=sides, flags=D.BIND_TIME_LAUNCHES)
        _fill(base.cfg, grads)
        red.sync(base.ready_order())
    torch.cuda.synchronize()
    assert red.buckets() == OP.compute_bucket_assignment_by_size(numels, 4, cap)
    assert red.launch_log() == closed_form_launch_log(red.buckets(), base.ready_order())
    with ThreadPoolExecutor(host_workers()) as pool:
        for v, n in enumerate(numels):
            bufs = [_regen_dev(base.cfg, r, v, n).cpu().numpy() for r in range(R)]
            want = to_device_f32(_oracle_mean(pool, bufs, np.empty(n, np.float32)))
            for r in range(R):
                assert_device_bits_equal(grads[r][v], want, f"blog v={v} r={r}")
    red.close()


def test_graph_replay_bert_large_every_element(bert_large_means, bert_large_grads):
    """A whole BERT-large sync captured into a HIP graph on the compute stream
    and replayed (the bench's --graph), twice, the inputs drawn again before
    each replay: every element of every replica against the oracle."""
    w = WC.BERT_LARGE
    numels = w.numels()
    P, R = len(numels), w.R
    say(f"{w.name} graph replay every element")
    compute, sides = _bench_streams()
    grads = bert_large_grads
    red = D.Reducer([p.shape for p in w.params()], R, w.cap_bytes)
    with torch.cuda.stream(compute):
        red.bind(grads, compute_stream=compute, side_streams=sides)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=compute):
        red.sync(w.ready_order())
    torch.cuda.synchronize()
    for rep in range(2):
        with torch.cuda.stream(compute):
            _fill(3, grads)
            g.replay()
        torch.cuda.synchronize()
        for v in range(P):
            want = to_device_f32(bert_large_means[v])
            for r in range(R):
                assert_device_bits_equal(grads[r][v], want, f"replay {rep} v={v} r={r}")
    red.close()


def test_bucket_view_bert_large_every_element(bert_large_means, bert_large_grads):
    """gradient_as_bucket_view at full size: the gradients are views of one flat
    storage per replica, as the bench's --mode view binds them."""
    w = WC.BERT_LARGE
    numels = w.numels()
    P, R = len(numels), w.R
    say(f"bucket view {w.name} every element")
    compute, sides = _bench_streams()
    red = D.Reducer([p.shape for p in w.params()], R, w.cap_bytes)
    with torch.cuda.stream(compute):
        views = red.bind_bucket_views(compute_stream=compute, side_streams=sides, flags=D.BIND_TIME_LAUNCHES)
        for r in range(R):
            for v, n in enumerate(numels):
                WG.normal(WG.seed_of(3, r, v), n, "cuda", out=views[r][v].view(-1))
        red.sync(w.ready_order())
    torch.cuda.synchronize()
    assert red.launch_log() == closed_form_launch_log(red.buckets(), w.ready_order())
    for v in range(P):
        want = to_device_f32(bert_large_means[v])
        for r in range(R):
            assert_device_bits_equal(views[r][v], want, f"view v={v} r={r}")
    red.close()


def test_unused_bert_large_every_element(bert_large_grads):
    """BERT-large shapes with some variables unused by single replicas and three
    unused by all of them (the bench's --unused-frac setup in spirit): every
    variable of every replica against a one-variable oracle reducer with the
    same flags (values are elementwise, so the bucketing does not change them)."""
    w = WC.BERT_LARGE
    numels = w.numels()
    P, R = len(numels), w.R
    used = np.ones((R, P), bool)
    for v in range(P):
        if v % 7 == 3:
            used[v % R, v] = False
        if v % 11 == 5:
            used[(v + 1) % R, v] = False
    for v in (5, 100, 389):
        used[:, v] = False
    G = used.any(axis=0)
    say(f"{w.name} unused: {int((~used).sum())} unused pairs, every element")
    compute, sides = _bench_streams()
    grads = bert_large_grads
    red = D.Reducer([p.shape for p in w.params()], R, w.cap_bytes)
    order = [v for v in w.ready_order() if G[v]]
    with torch.cuda.stream(compute):
        red.bind(grads, compute_stream=compute, side_streams=sides, flags=D.BIND_TIME_LAUNCHES)
        _fill(3, grads)
        red.set_local_used(used)
        red.sync(order)
    torch.cuda.synchronize()
    assert [b for b, _ in red.launch_log()] == list(range(red.num_buckets))

    stage = HostStage(R, max(numels))
    out = HostStage(R, max(numels))
    with ThreadPoolExecutor(host_workers()) as pool:
        for v, n in enumerate(numels):
            _progress(v, P, "unused oracle")
            bufs = [stage.fetch(r, _regen_dev(3, r, v, n)) for r in range(R)]
            want = [out.bufs[r][:n] for r in range(R)]

            def job(ab, v=v, bufs=bufs, want=want):
                a, b = ab
                orc = OR.Reducer([b - a], R, 0)
                og = [[bufs[r][a:b].copy()] for r in range(R)]
                orc.bind(og)
                orc.set_local_used(used[:, v:v + 1])
                orc.sync([0] if G[v] else [])
                for r in range(R):
                    want[r][a:b] = og[r][0]

            list(pool.map(job, _chunks(n)))
            for r in range(R):
                assert_device_bits_equal(grads[r][v], want[r], f"unused v={v} r={r}")
    red.close()


# --- config 4: no_sync, BERT-base shapes, R = 16, k = 8 bf16 micro-steps -------------

@pytest.fixture(scope="module")
def nosync_expected():
    """The oracle's result of config 4: k bf16 micro-steps accumulated in fp32
    per replica, then one synchronisation. The step gradients are drawn again
    per replica and micro-step, as the run drew them, and kept on the device;
    every variable is cut into element chunks, each an independent one-variable
    oracle reducer on a host thread (values are elementwise, so the split
    changes no bit), fed from a reused host staging slot."""
    import queue
    w = WC.BERT_BASE_NOSYNC
    numels = w.numels()
    P, R, k = len(numels), w.R, w.micro_steps
    N = sum(numels)
    offs = np.concatenate([[0], np.cumsum(numels)]).astype(np.int64)
    chunk = 1 << 18
    pieces = [(v, a, b) for v in range(P) for a, b in _chunks(numels[v], chunk)]
    nthr = host_workers()
    say(f"oracle for {w.name}: R={R} k={k}, {len(pieces)} chunks on {nthr} host threads")
    flats = [[WG.flat_step(4, r, t, N, "cuda").view(torch.int16) for r in range(R)] for t in range(k)]
    slots = queue.Queue()
    for _ in range(nthr + 2):
        slots.put(np.empty((k, R, chunk), np.uint16))
    want = {v: np.empty(n, np.float32) for v, n in enumerate(numels)}

    def job(piece, slot):
        v, a, b = piece
        orc = OR.Reducer([b - a], R, 0)
        acc = [[np.zeros(b - a, np.float32)] for _ in range(R)]
        orc.bind(acc)
        orc.set_sync(False)
        for t in range(k):
            orc.no_sync_accumulate([[slot[t, r, :b - a]] for r in range(R)], first=(t == 0))
        orc.set_sync(True)
        orc.sync()
        for r in range(1, R):                  # the oracle wrote one mean to every replica
            assert np.array_equal(acc[r][0].view(np.uint32), acc[0][0].view(np.uint32))
        want[v][a:b] = acc[0][0]
        slots.put(slot)

    with ThreadPoolExecutor(nthr) as pool:
        futs = []
        for i, piece in enumerate(pieces):
            _progress(i, len(pieces), "no_sync oracle chunks")
            v, a, b = piece
            o = int(offs[v])
            slot = slots.get()
            for t in range(k):
                for r in range(R):
                    torch.from_numpy(slot[t, r, :b - a].view(np.int16)).copy_(flats[t][r][o + a:o + b])
            futs.append(pool.submit(job, piece, slot))
        for f in futs:
            f.result()
    del flats
    say("oracle no_sync result ready")
    return want


@pytest.mark.parametrize("fused_last_step", [False, True])
def test_config4_nosync_every_element(fused_last_step, nosync_expected):
    """The bench's no_sync step: k-1 micro-steps accumulated with sync off, the
    k-th with sync on (accumulated by its own pass, or by the reduction itself
    through ddpb_set_sync_step), every element of all 16 replicas."""
    w = WC.BERT_BASE_NOSYNC
    numels = w.numels()
    P, R, k = len(numels), w.R, w.micro_steps
    N = sum(numels)
    say(f"{w.name}: every element, fused_last_step={fused_last_step}")
    compute, sides = _bench_streams()
    grads = alloc_grads(numels, R)
    red = D.Reducer([p.shape for p in w.params()], R, w.cap_bytes)
    assert red.num_buckets == 13
    order = w.ready_order()
    with torch.cuda.stream(compute):
        red.bind(grads, compute_stream=compute, side_streams=sides, flags=D.BIND_TIME_LAUNCHES)
        red.set_sync(False)
        for t in range(k):
            flats = [WG.flat_step(4, r, t, N, "cuda") for r in range(R)]
            table = red.step_table([WG.flat_views(f, numels) for f in flats])
            if t == k - 1:
                red.set_sync(True)
                if fused_last_step:
                    red.set_sync_step(table, first_step=(t == 0))
                    red.sync(order)
                    torch.cuda.synchronize()       # the step memory is read until finalize's join
                    break
            red.no_sync_accumulate(table, first_step=(t == 0))
            red.sync(order)                        # no-ops until the last micro-step
            torch.cuda.synchronize()               # before this micro-step's draws are freed
    torch.cuda.synchronize()
    assert red.launch_log() == closed_form_launch_log(red.buckets(), order)
    for v in range(P):
        want = to_device_f32(nosync_expected[v])
        for r in range(R):
            assert_device_bits_equal(grads[r][v], want, f"fused={fused_last_step} v={v} r={r}")
    red.close()


# --- config 5: overlap with a bf16 MLP backward ------------------------------------

def _mlp_backward(g0, X, H, W1, W2, dY0, hook):
    """Backward of [Linear(d, f), Linear(f, d)] blocks in bf16, last layer
    first; fp32 gradients of replica 0 are written in place, each followed by
    its hook."""
    L = len(X)
    dY = dY0
    for l in range(L - 1, -1, -1):
        vW1, vb1, vW2, vb2 = 4 * l, 4 * l + 1, 4 * l + 2, 4 * l + 3
        torch.sum(dY, dim=0, dtype=torch.float32, out=g0[vb2])
        hook(vb2)
        torch.mm(dY.t(), H[l], torch.float32, out=g0[vW2])
        hook(vW2)
        dH = torch.mm(dY, W2[l])
        torch.sum(dH, dim=0, dtype=torch.float32, out=g0[vb1])
        hook(vb1)
        torch.mm(dH.t(), X[l], torch.float32, out=g0[vW1])
        hook(vW1)
        dY = torch.mm(dH, W1[l])


@pytest.mark.parametrize("size,wg", [("small", 1), ("full", 1), ("full", 0)])
def test_config5_overlap_every_element(size, wg):
    """Replica 0's gradients come from a bf16 backward on the compute stream,
    layer by layer, each hook right after its gradient is written; buckets are
    reduced on two side streams meanwhile. Every variable of every replica is
    compared with the oracle's mean of replica 0's pre-hook snapshot and the
    resident replicas 1..7."""
    if size == "small":
        L, d, f, T, cap = 3, 256, 1024, 512, 4 * 300000
    else:
        L, d, f, T, cap = 24, 2048, 8192, 8192, WC.MLP_OVERLAP.cap_bytes
    params = WS.mlp(L, d, f)
    numels = WS.numels(params)
    P, R = len(numels), 8
    say(f"config5 {size}: L={L} d={d} f={f} T={T} P={P} workgroups_per_cu={wg}")
    comp, sides = _bench_streams()
    with torch.cuda.stream(comp):
        grads = alloc_grads(numels, R)
        snap = [torch.empty(n, dtype=torch.float32, device="cuda") for n in numels]
        for r in range(1, R):
            for v, n in enumerate(numels):
                WG.normal(WG.seed_of(5, r, v), n, "cuda", out=grads[r][v])
        g = torch.Generator(device="cuda").manual_seed(5)
        bf = torch.bfloat16
        X = [torch.randn(T, d, device="cuda", dtype=bf, generator=g) for _ in range(L)]
        H = [torch.randn(T, f, device="cuda", dtype=bf, generator=g) for _ in range(L)]
        W1 = [torch.randn(f, d, device="cuda", dtype=bf, generator=g) * 0.02 for _ in range(L)]
        W2 = [torch.randn(d, f, device="cuda", dtype=bf, generator=g) * 0.02 for _ in range(L)]
        dY0 = torch.randn(T, d, device="cuda", dtype=bf, generator=g)
        red = D.Reducer([p.shape for p in params], R, cap)
        red.bind(grads, compute_stream=comp, side_streams=sides, flags=D.BIND_TIME_LAUNCHES)
        red.set_workgroups_per_cu(wg)
        g0 = [grads[0][v].view(params[v].shape) for v in range(P)]

        def hook(v):
            snap[v].copy_(grads[0][v])          # on the compute stream, before the ready event
            red.mark_ready(v)

        _mlp_backward(g0, X, H, W1, W2, dY0, hook)
        red.finalize()
    torch.cuda.synchronize()
    order = list(range(P))[::-1]                   # the backward's hook order
    assert red.launch_log() == closed_form_launch_log(red.buckets(), order)
    stage = HostStage(R, max(numels))
    out = np.empty(max(numels), np.float32)
    with ThreadPoolExecutor(host_workers()) as pool:
        for v, n in enumerate(numels):
            _progress(v, P, "config5 oracle")
            bufs = [stage.fetch(0, snap[v])] + [stage.fetch(r, _regen_dev(5, r, v, n)) for r in range(1, R)]
            want = to_device_f32(_oracle_mean(pool, bufs, out[:n]))
            for r in range(R):
                assert_device_bits_equal(grads[r][v], want, f"config5 {size} v={v} r={r}")
    red.close()


def test_config5_rebuilt_from_shuffled_order_every_element():
    """The bench's --config 5 --shuffle-params --rebuild at full size: the 96
    parameters are defined in a seeded shuffled order, a first iteration runs
    as one bucket and records the hook order, the buckets are rebuilt from it
    (same cap) and bound again, and the second iteration's overlapped backward
    is checked on every element of every replica against the oracle, with
    replica 0 snapshotted on the compute stream before each hook."""
    L, d, f, T, cap = 24, 2048, 8192, 8192, WC.MLP_OVERLAP.cap_bytes
    params = WS.mlp(L, d, f)
    numels = WS.numels(params)
    P, R = len(numels), 8
    perm = WG.permutation(55, P)                 # definition index k holds layer-order variable perm[k]
    dpos = [0] * P
    for k, v in enumerate(perm):
        dpos[v] = k
    say(f"config5 shuffled + rebuild: P={P} R={R}")
    comp, sides = _bench_streams()
    with torch.cuda.stream(comp):
        grads = alloc_grads(numels, R)           # layer-order variables
        snap = [torch.empty(n, dtype=torch.float32, device="cuda") for n in numels]
        g = torch.Generator(device="cuda").manual_seed(5)
        bf = torch.bfloat16
        X = [torch.randn(T, d, device="cuda", dtype=bf, generator=g) for _ in range(L)]
        H = [torch.randn(T, f, device="cuda", dtype=bf, generator=g) for _ in range(L)]
        W1 = [torch.randn(f, d, device="cuda", dtype=bf, generator=g) * 0.02 for _ in range(L)]
        W2 = [torch.randn(d, f, device="cuda", dtype=bf, generator=g) * 0.02 for _ in range(L)]
        dY0 = torch.randn(T, d, device="cuda", dtype=bf, generator=g)
        shapes_def = [params[v].shape for v in perm]
        grads_def = [[row[v] for v in perm] for row in grads]
        red = D.Reducer(shapes_def, R, 1 << 62)
        red.bind(grads_def, compute_stream=comp, side_streams=sides, flags=D.BIND_TIME_LAUNCHES | D.BIND_OVERLAP)
        g0 = [grads[0][v].view(params[v].shape) for v in range(P)]

        def fill_peers():
            for r in range(1, R):
                for v, n in enumerate(numels):
                    WG.normal(WG.seed_of(5, r, v), n, "cuda", out=grads[r][v])

        fill_peers()
        _mlp_backward(g0, X, H, W1, W2, dY0, lambda v: red.mark_ready(dpos[v]))
        red.finalize()
        assert red.num_buckets == 1
        red.rebuild_buckets(cap)
        red.bind(grads_def, compute_stream=comp, side_streams=sides, flags=D.BIND_TIME_LAUNCHES | D.BIND_OVERLAP)
        fill_peers()                             # the first iteration averaged them

        def hook(v):
            snap[v].copy_(grads[0][v])
            red.mark_ready(dpos[v])

        _mlp_backward(g0, X, H, W1, W2, dY0, hook)
        red.finalize()
    torch.cuda.synchronize()
    hook_order = [dpos[v] for v in range(P)][::-1]     # definition indices in the backward's order
    want_buckets = OP.compute_bucket_assignment_by_size([numels[v] for v in perm], 4, cap, order=hook_order)
    assert red.buckets() == want_buckets and red.num_buckets == 48
    assert red.launch_log() == closed_form_launch_log(want_buckets, hook_order)
    stage = HostStage(R, max(numels))
    out = np.empty(max(numels), np.float32)
    with ThreadPoolExecutor(host_workers()) as pool:
        for v, n in enumerate(numels):
            _progress(v, P, "rebuilt config5 oracle")
            bufs = [stage.fetch(0, snap[v])] + [stage.fetch(r, _regen_dev(5, r, v, n)) for r in range(1, R)]
            want = to_device_f32(_oracle_mean(pool, bufs, out[:n]))
            for r in range(R):
                assert_device_bits_equal(grads[r][v], want, f"rebuilt v={v} r={r}")
    red.close()
