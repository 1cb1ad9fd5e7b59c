"""CPU tests of the native host core through the C ABI: the library loads and
exports every declared symbol; the plan, locators and segment table agree with
the oracle; the readiness state machine launches exactly as the oracle does;
error codes behave as documented.

The state machine runs in the host-only test build (same core.cpp/abi.cpp,
launcher that enqueues nothing), so no GPU is needed.
"""
import os
import re

import numpy as np
import pytest

import ddp_bucketed_gradient_amd as D
from ddp_bucketed_gradient_amd import _abi
from oracle import plan as OP
from oracle import reducer as OR
from workloads import shapes as WS, gen as WG

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddpb.h")
MiB = 1 << 20


@pytest.fixture(scope="module")
def host():
    if not os.path.exists(D.HOSTONLY_LIB):
        from ddp_bucketed_gradient_amd import build
        build.build_hostonly()
    return D.Lib(D.HOSTONLY_LIB)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddpb_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(_abi.SYMBOLS)


@pytest.mark.parametrize("path", [D.HIP_LIB, D.HOSTONLY_LIB])
def test_library_loads_and_exports_every_symbol(path, host):
    if not os.path.exists(path):
        pytest.skip(f"{path} not built")
    lib = D.Lib(path)
    for name in _declared():
        assert hasattr(lib.dll, name), name


def _reducer(host, numels, R, cap):
    return D.Reducer([(n,) for n in numels], R, cap, lib=host)


def _bind_fake(red):
    # the host-only launcher never dereferences pointers; any non-null value
    red.bind_ptrs([0x1000 + 16 * i for i in range(red.R * red.P)], side_streams=[0])


# --- plan -----------------------------------------------------------------------

PLAN_CASES = [
    (WS.numels(WS.linear10()), 25 * MiB),
    (WS.numels(WS.resnet50()), 25 * MiB),
    (WS.numels(WS.bert_large()), 25 * MiB),
    (WS.numels(WS.bert_large()), 0),
    (WS.numels(WS.bert_large()), 1 * MiB),
    (WS.numels(WS.bert_large()), 200 * MiB),
    (WS.numels(WS.bert_base()), 25 * MiB),
    (WS.numels(WS.mlp()), 25 * MiB),
    (WS.numels(WS.blog_fine1()), 4 * MiB),
    (WS.numels(WS.blog_coarse4()), 64 * MiB),
    ([], 25 * MiB),
    ([0, 5, 0, 7], 0),
]


@pytest.mark.parametrize("numels,cap", PLAN_CASES)
def test_plan_and_locators_match_oracle(host, numels, cap):
    red = _reducer(host, numels, 2, cap)
    want = OP.compute_bucket_assignment_by_size(numels, 4, cap)
    assert red.buckets() == want
    assert red.bucket_bytes() == [4 * x for x in OP.bucket_numels(want, numels)]
    loc = OP.locators(want, numels)
    for v in range(len(numels)):
        assert red.locator(v) == (loc[v].bucket, loc[v].intra, loc[v].offset, loc[v].length)


@pytest.mark.parametrize("seed", range(25))
def test_plan_random_matches_oracle(host, seed):
    rng = np.random.default_rng(seed)
    numels = WG.random_numels(seed, int(rng.integers(1, 60)), 0, 20000)
    cap = int(rng.integers(0, 4 * sum(numels) + 10))
    red = _reducer(host, numels, 3, cap)
    assert red.buckets() == OP.compute_bucket_assignment_by_size(numels, 4, cap)


@pytest.mark.parametrize("numels,cap", PLAN_CASES[:8])
def test_segment_table_covers_every_variable_once(host, numels, cap):
    red = _reducer(host, numels, 2, cap)
    nseg, seg_elems = host.num_segments(red.h)
    assert seg_elems >= 64 and seg_elems % 64 == 0
    buckets = red.buckets()
    seen = 0
    for b, members in enumerate(buckets):
        first, count = host.get_bucket_segments(red.h, b)
        assert first == seen
        segs = [host.get_segment(red.h, first + i) for i in range(count)]
        k = 0
        for v in members:
            _, _, off, n = red.locator(v)
            start = 0
            while start < n:
                var, bb, st, ln, bo = segs[k]
                assert (var, bb, st, bo) == (v, b, start, off + start)
                assert 0 < ln <= seg_elems and (ln == seg_elems or start + ln == n)
                start += ln
                k += 1
        assert k == count
        seen += count
    assert seen == nseg
    assert nseg == sum((n + seg_elems - 1) // seg_elems for n in numels)


def test_plan_of_a_tensor_beyond_int32_elements(host):
    """A tensor of 2^31 + 9221 elements: locators, the segments that start at
    and past 2^31, and the staged workspace are 64-bit throughout."""
    big = (1 << 31) + 9221
    numels = [5, big, 7]
    for cap in (25 * MiB, 0):
        red = _reducer(host, numels, 2, cap)
        want = OP.compute_bucket_assignment_by_size(numels, 4, cap)
        assert red.buckets() == want
        loc = OP.locators(want, numels)
        for v in range(3):
            assert red.locator(v) == (loc[v].bucket, loc[v].intra, loc[v].offset, loc[v].length)
        nseg, E = host.num_segments(red.h)
        assert nseg == 1 + (big + E - 1) // E + 1
        b1, _, off1, _ = red.locator(1)
        first, count = host.get_bucket_segments(red.h, b1)
        k0 = first + (1 if cap else 0)                # the 7-element variable comes first at 25 MiB
        at_edge = host.get_segment(red.h, k0 + (1 << 31) // E)
        assert at_edge == (1, b1, 1 << 31, E, off1 + (1 << 31))
        last = host.get_segment(red.h, k0 + (big - 1) // E)
        assert last == (1, b1, (big - 1) // E * E, big - (big - 1) // E * E, off1 + (big - 1) // E * E)
        flat = sum((n + 63) // 64 * 64 for n in OP.bucket_numels(want, numels))
        assert red.workspace_bytes(D.MODE_STAGED) == 3 * flat * 4
        assert host.view_storage_elems(red.h) == flat


def test_sync_step_rules(host):
    """ddpb_set_sync_step: bound, before the iteration's hooks, with sync on;
    consumed by finalize, dropped by reset; sync cannot be turned off while
    it is set."""
    red = _reducer(host, [10, 20], 2, 0)
    fake = [0x2000 + 16 * i for i in range(4)]

    def code(fn):
        with pytest.raises(D.DdpbError) as e:
            fn()
        return e.value.code

    assert code(lambda: host.set_sync_step(red.h, fake, D.BF16, False)) == D.E_STATE      # not bound
    _bind_fake(red)
    assert code(lambda: host.set_sync_step(red.h, fake, 7, False)) == D.E_ARG             # bad dtype
    host.set_sync_step(red.h, fake, D.BF16, False)
    assert code(lambda: red.set_sync(False)) == D.E_STATE                                 # step pending
    red.mark_ready(1)
    assert code(lambda: host.set_sync_step(red.h, fake, D.BF16, False)) == D.E_STATE      # iteration open
    red.mark_ready(0)
    red.finalize()
    red.set_sync(False)                                                                   # consumed
    assert code(lambda: host.set_sync_step(red.h, fake, D.F32, True)) == D.E_STATE        # sync off
    red.set_sync(True)
    host.set_sync_step(red.h, fake, D.F32, True)
    red.reset()
    red.set_sync(False)                                                                   # dropped by reset
    red.set_sync(True)
    host.set_sync_step(red.h, fake, D.F32, False)
    _bind_fake(red)
    red.set_sync(False)                                                                   # dropped by a rebind


def test_workgroups_per_cu_arguments(host):
    red = _reducer(host, [10, 20], 2, 0)
    for n in (0, 1, 2):
        red.set_workgroups_per_cu(n)
    for n in (-1, 3):
        with pytest.raises(D.DdpbError) as e:
            red.set_workgroups_per_cu(n)
        assert e.value.code == D.E_ARG


def test_workspace_bytes(host):
    numels = [10, 100, 3]
    red = _reducer(host, numels, 4, 0)
    assert red.workspace_bytes(D.MODE_FUSED) == 0
    # three one-tensor buckets padded to 64 elements each, R + 1 copies
    assert red.workspace_bytes(D.MODE_STAGED) == (4 + 1) * (64 + 128 + 64) * 4


# --- readiness state machine vs the oracle ------------------------------------------

@pytest.mark.parametrize("seed", range(30))
def test_launch_log_matches_oracle_random_orders(host, seed):
    rng = np.random.default_rng(100 + seed)
    P = int(rng.integers(1, 40))
    numels = WG.random_numels(seed, P, 1, 64)
    cap = int(rng.integers(0, 4 * sum(numels) // 3 + 1))
    orc = OR.Reducer(numels, 2, cap)
    orc.bind([[np.zeros(n, np.float32) for n in numels] for _ in range(2)])
    red = _reducer(host, numels, 2, cap)
    _bind_fake(red)
    for it in range(3):                      # several iterations in a row
        order = WG.permutation(seed * 10 + it, P)
        orc.launch_log.clear()
        orc.sync(order)
        red.sync(order)
        assert red.launch_log() == orc.launch_log


def test_printed_in_order_sequence_native(host):
    red = _reducer(host, [4, 4, 4], 2, 0)
    _bind_fake(red)
    red.mark_ready(2)
    assert red.launch_log() == [(0, 0)]
    red.mark_ready(0)                        # bucket 2 completes first: parked
    assert red.launch_log() == [(0, 0)]
    red.mark_ready(1)                        # bucket 1, then the parked bucket 2
    assert red.launch_log() == [(0, 0), (1, 2), (2, 2)]
    red.finalize()


def test_mark_ready_many_equals_single_calls(host):
    numels = WG.random_numels(5, 30, 1, 100)
    order = WG.permutation(5, 30)
    a, b = _reducer(host, numels, 2, 400), _reducer(host, numels, 2, 400)
    _bind_fake(a)
    _bind_fake(b)
    a.sync(order)
    b.mark_ready_many(order)
    b.finalize()
    assert a.launch_log() == b.launch_log()


# --- errors ----------------------------------------------------------------------------

def _code(fn, *a):
    try:
        fn(*a)
    except D.DdpbError as e:
        return e.code
    return 0


def test_errors(host):
    red = _reducer(host, [4, 4, 4], 2, 0)
    assert _code(red.mark_ready, 0) == _abi.E_STATE          # not bound
    _bind_fake(red)
    assert _code(red.mark_ready, 3) == _abi.E_INDEX
    assert _code(red.mark_ready, -1) == _abi.E_INDEX
    red.mark_ready(2)
    assert _code(red.mark_ready, 2) == _abi.E_DOUBLE_READY
    assert _code(red.set_sync, False) == _abi.E_STATE        # mid-iteration
    red.mark_ready(1)                                        # variable 0 never arrives
    assert _code(red.finalize) == _abi.E_INCOMPLETE
    assert "prior iteration" in host.last_error() or "not every bucket" in host.last_error()
    assert _code(red.mark_ready, 2) == _abi.E_INCOMPLETE     # latched
    assert _code(red.ensure_prior_reduction_finished) == _abi.E_INCOMPLETE
    red.reset()
    red.ensure_prior_reduction_finished()
    red.sync()
    assert red.launch_log() == [(0, 0), (1, 1), (2, 2)]


def test_unfinished_iteration_detected_before_next_forward(host):
    red = _reducer(host, [4, 4], 2, 0)
    _bind_fake(red)
    red.mark_ready(1)
    assert _code(red.ensure_prior_reduction_finished) == _abi.E_INCOMPLETE
    assert "previous iteration left buckets unreduced" in host.last_error()


def test_create_argument_errors(host):
    assert _code(host.reducer_create, [(4,)], D.F32, 0, 0) == _abi.E_ARG          # R = 0
    assert _code(host.reducer_create, [(4,)], D.F32, 0, 65) == _abi.E_ARG         # R too large
    assert _code(host.reducer_create, [(4,)], D.F32, -1, 2) == _abi.E_ARG         # negative cap
    assert _code(host.reducer_create, [(4,)], D.BF16, 0, 2) == _abi.E_ARG         # fp32 only
    assert _code(host.reducer_create, [(4, -1)], D.F32, 0, 2) == _abi.E_ARG       # negative dim
    h = host.reducer_create([(), (2, 3)], D.F32, 0, 2)                             # scalar param
    assert host.get_locator(h, 0)[3] == 1 and host.get_locator(h, 1)[3] == 6
    host.destroy(h)


def test_bind_argument_errors(host):
    red = _reducer(host, [4, 4], 2, 0)
    ptrs = [0x1000] * 4
    assert _code(red.bind_ptrs, ptrs, 0, 0, 0, []) == _abi.E_ARG                  # no side stream
    assert _code(red.bind_ptrs, [0] * 4) == _abi.E_ARG                            # null gradient
    assert _code(red.bind_ptrs, ptrs, 0, 0, 0, [0], 1) == _abi.E_ARG              # staged needs workspace
    assert _code(red.bind_ptrs, ptrs, 0, 0, 0, [0], 7) == _abi.E_ARG              # bad mode
    red.bind_ptrs(ptrs)
    red.mark_ready(1)
    assert _code(red.bind_ptrs, ptrs) == _abi.E_STATE                             # mid-iteration


def test_no_sync_makes_hooks_noops(host):
    red = _reducer(host, [4, 4, 4], 2, 0)
    _bind_fake(red)
    red.set_sync(False)
    red.sync()                                   # hooks run, nothing launches
    assert red.launch_log() == []
    red.finalize()                               # no-op
    red.set_sync(True)
    red.sync()
    assert [b for b, _ in red.launch_log()] == [0, 1, 2]


def test_empty_model(host):
    red = _reducer(host, [], 4, 25 * MiB)
    assert red.num_buckets == 0
    red.bind_ptrs([], side_streams=[0])
    red.finalize()


def test_binding_checks_step_tensors_before_the_library_sees_them(host):
    """A step tensor of the wrong size, dtype or device never reaches the
    kernels: the binding raises first (CPU tensors stand in for the wrong
    device here)."""
    import torch
    red = D.Reducer([(4,), (6,)], 2, 0, lib=host)
    _bind_fake(red)
    ok = [[torch.zeros(4), torch.zeros(6)] for _ in range(2)]
    with pytest.raises(ValueError):
        red.no_sync_accumulate(ok, True)                      # not CUDA tensors
    with pytest.raises(ValueError):
        red.no_sync_accumulate([[torch.zeros(4, dtype=torch.float16), None]] * 2, True)


def test_failed_rebuild_keeps_the_cap(host):
    red = D.Reducer([(4,), (6,)], 2, 8, lib=host)
    _bind_fake(red)
    with pytest.raises(D.DdpbError):
        red.rebuild_buckets(0)                                # no finished iteration yet
    assert red.cap == 8


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: without the built library the binding raises."""
    with pytest.raises(ImportError, match="no fallback"):
        D.Lib(str(tmp_path / "libddpb.so"))


def test_pointer_array_marshalling(host):
    """The binding's void* arrays: addresses in order, 0 as NULL, never empty;
    a prebuilt array is accepted wherever a list of addresses is."""
    from ddp_bucketed_gradient_amd import _abi
    a = _abi.ptr_array([0x1000, 0, 0x2010])
    assert len(a) == 3 and [a[0], a[1], a[2]] == [0x1000, None, 0x2010]
    assert len(_abi.ptr_array([])) == 1
    red = _reducer(host, [10, 20], 2, 0)
    _bind_fake(red)
    fake = [0x2000 + 16 * i for i in range(4)]
    host.set_sync_step(red.h, _abi.ptr_array(fake), D.BF16, False)
    red.reset()
    host.no_sync_accumulate(red.h, _abi.ptr_array(fake), D.F32, True)


def test_step_table_checks_before_the_library(host):
    """Reducer.step_table refuses a wrong R x P layout, a wrong element count,
    mixed dtypes and host tensors before any address reaches the library."""
    import torch
    red = _reducer(host, [4, 6], 2, 0)
    ok = [[torch.zeros(4), torch.zeros(6)] for _ in range(2)]
    with pytest.raises(ValueError):
        red.step_table(ok[:1])                                   # one replica short
    with pytest.raises(ValueError):
        red.step_table([[torch.zeros(4)] for _ in range(2)])     # one variable short
    with pytest.raises(ValueError):
        red.step_table(ok)                                       # not CUDA tensors
    with pytest.raises(ValueError):
        red.step_table([[torch.zeros(4, dtype=torch.float16), None] for _ in range(2)])   # not fp32 / bf16
    t = red.step_table([[None, None] for _ in range(2)])         # no step anywhere: all NULL
    assert [t.ptrs[i] for i in range(4)] == [None] * 4 and t.code == D.F32


def test_bind_flags(host):
    """ddpb_bind takes DDPB_BIND_DEVICE_TIMESTAMPS, DDPB_BIND_TIME_LAUNCHES,
    DDPB_BIND_ROCTX and DDPB_BIND_OVERLAP in any combination and refuses
    unknown bits."""
    red = _reducer(host, [10, 20], 2, 0)
    ptrs = [0x1000 + 16 * i for i in range(4)]
    for f in (0, D.BIND_DEVICE_TIMESTAMPS, D.BIND_TIME_LAUNCHES, D.BIND_ROCTX, D.BIND_OVERLAP,
              D.BIND_DEVICE_TIMESTAMPS | D.BIND_TIME_LAUNCHES | D.BIND_ROCTX | D.BIND_OVERLAP):
        red.bind_ptrs(ptrs, side_streams=[0], flags=f)
        red.sync()
    for bad in (16, 1 << 20, -1):
        with pytest.raises(D.DdpbError) as e:
            red.bind_ptrs(ptrs, side_streams=[0], flags=bad)
        assert e.value.code == D.E_ARG


def _joins(host):
    f = host.dll.ddpb_hostonly_join_count
    f.restype = __import__("ctypes").c_longlong
    return f()


def test_accumulate_refused_inside_an_open_or_failed_iteration(host):
    """A local backward's accumulation runs on the compute stream; inside an
    open iteration (buckets may still be reducing on the side streams) it is
    refused, and while a failed iteration is latched it fails like the hooks.
    The oracle refuses the same way."""
    from oracle import reducer as OR
    numels = [4, 4, 4]
    red = _reducer(host, numels, 2, 16)
    _bind_fake(red)
    orc = OR.Reducer(numels, 2, 16)
    orc.bind([[np.zeros(n, np.float32) for n in numels] for _ in range(2)])
    steps = [[np.zeros(n, np.float32) for n in numels] for _ in range(2)]
    fake = _abi.ptr_array([0x3000 + 64 * i for i in range(2 * len(numels))])
    red.mark_ready(2)
    orc.mark_ready(2)
    with pytest.raises(D.DdpbError) as e:
        host.no_sync_accumulate(red.h, fake, D.F32, False)
    assert e.value.code == _abi.E_STATE
    with pytest.raises(RuntimeError):
        orc.no_sync_accumulate(steps, first=False)
    for side in (red.finalize, orc.finalize):
        with pytest.raises((D.DdpbError, OR.ReductionIncomplete)):
            side()
    with pytest.raises(D.DdpbError) as e:
        host.no_sync_accumulate(red.h, fake, D.F32, False)
    assert e.value.code == _abi.E_INCOMPLETE
    with pytest.raises(OR.ReductionIncomplete):
        orc.no_sync_accumulate(steps, first=False)
    with pytest.raises(D.DdpbError) as e:
        host.set_sync_step(red.h, fake, D.F32, False)
    assert e.value.code == _abi.E_INCOMPLETE
    red.reset()
    orc.reset()
    host.no_sync_accumulate(red.h, fake, D.F32, False)
    orc.no_sync_accumulate(steps, first=False)


def test_reset_and_failed_finalize_join_the_side_streams(host):
    """Buckets launched before a failure keep running; a failed finalize and a
    reset make the compute stream wait for the side streams so that later work
    cannot race with their copy-back."""
    red = _reducer(host, [4, 4, 4], 2, 16)
    _bind_fake(red)
    red.mark_ready(2)                            # bucket 0 launches
    j0 = _joins(host)
    with pytest.raises(D.DdpbError):
        red.finalize()
    assert _joins(host) == j0 + 1
    red.reset()
    assert _joins(host) == j0 + 2
    red.sync()
    assert _joins(host) == j0 + 3


def test_reset_drops_used_flags(host):
    """Used flags belong to the synchronisation they were set for; after a
    failed iteration and a reset, the next iteration expects every variable
    again (stale flags would mark variable 1 ready by themselves and refuse its
    hook as a double ready). The oracle agrees."""
    from oracle import reducer as OR
    numels = [4, 4]
    red = _reducer(host, numels, 2, 0)
    _bind_fake(red)
    orc = OR.Reducer(numels, 2, 0)
    orc.bind([[np.zeros(n, np.float32) for n in numels] for _ in range(2)])
    used = [[True, False], [True, False]]
    red.set_local_used(used)
    orc.set_local_used(used)
    red.mark_ready(0)
    orc.mark_ready(0)
    red.reset()                                   # abandon it: the flags go with it
    orc.reset()
    red.sync([1, 0])
    orc.sync([1, 0])
    assert red.launch_log() == orc.launch_log[-2:] == [(0, 0), (1, 1)]


def test_static_binding_arguments_and_refusals(host):
    """ddpb_bind_static: bad mode and NULL gradient pointers are refused before
    anything is bound; on a static binding the calls that need pinned staging
    (accumulation, synchronising step, used flags) are refused, syncs run; a
    later ddpb_bind lifts the refusals."""
    red = _reducer(host, [4, 6], 2, 0)
    ptrs = [0x1000 + 64 * i for i in range(4)]
    with pytest.raises(D.DdpbError) as e:
        host.bind_static(red.h, ptrs, 0, 7)
    assert e.value.code == _abi.E_ARG
    with pytest.raises(D.DdpbError) as e:
        host.bind_static(red.h, ptrs[:3] + [0], 0, D.MODE_FUSED)
    assert e.value.code == _abi.E_ARG
    host.bind_static(red.h, ptrs, 0, D.MODE_STAGED)
    fake = _abi.ptr_array([0x5000 + 64 * i for i in range(4)])
    for call in (lambda: host.no_sync_accumulate(red.h, fake, D.F32, True),
                 lambda: host.set_sync_step(red.h, fake, D.F32, False),
                 lambda: host.set_local_used(red.h, [1, 1, 1, 0])):
        with pytest.raises(D.DdpbError) as e:
            call()
        assert e.value.code == _abi.E_STATE
    red.sync()
    assert red.launch_log() == [(0, 0), (1, 1)]
    _bind_fake(red)
    host.no_sync_accumulate(red.h, fake, D.F32, True)
