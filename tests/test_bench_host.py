"""CPU tests of the bench's host-side logic: the busy-time union of launch
intervals, the traffic lookup keyed by the kernel sources' hash, and the
refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("starts,durs,want", [
    ([], [], 0.0),
    ([0.0], [2.0], 2.0),
    ([0.0, 5.0], [2.0, 1.0], 3.0),            # disjoint
    ([0.0, 1.0], [2.0, 2.0], 3.0),            # overlapping
    ([0.0, 0.5], [3.0, 1.0], 3.0),            # nested
    ([4.0, 0.0, 1.0], [1.0, 2.0, 2.0], 4.0),  # unsorted, touching
])
def test_union_length(starts, durs, want):
    assert bench.union_length(starts, durs) == pytest.approx(want)


def test_union_length_matches_brute_force():
    import random
    rng = random.Random(3)
    for _ in range(200):
        n = rng.randint(1, 12)
        st = [rng.randint(0, 40) for _ in range(n)]
        du = [rng.randint(0, 10) for _ in range(n)]
        covered = set()
        for s, d in zip(st, du):
            covered.update(range(s, s + d))
        assert bench.union_length(st, du) == pytest.approx(len(covered))


def test_traffic_only_for_the_measured_kernels(tmp_path, monkeypatch):
    """A stored counter figure is reported only while the built device code is
    the one measured (its hash), or, for an entry without one, while the
    kernel sources are."""
    from ddp_bucketed_gradient_amd import profiling as PF
    key = "fused_mean_kernel:some_workload"
    prof = tmp_path / "profiles"
    prof.mkdir()
    entry = {"device_code_sha256_16": "ab" * 8, "bytes_per_launch": 1234}
    old = {"kernel_source_sha256_16": "cd" * 8, "bytes_per_launch": 99}
    (prof / "traffic.json").write_text(json.dumps({key: entry, "k:old": old}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(PF, "device_code_hash", lambda lib_path=None: "ab" * 8)
    monkeypatch.setattr(PF, "kernel_source_hash", lambda: "cd" * 8)
    assert bench.traffic_from_profiles("fused_mean_kernel", "some_workload") == 1234
    assert bench.traffic_from_profiles("fused_mean_kernel", "other_workload") is None
    assert bench.traffic_from_profiles("k", "old") == 99
    monkeypatch.setattr(PF, "device_code_hash", lambda lib_path=None: "0" * 16)    # kernels rebuilt since
    monkeypatch.setattr(PF, "kernel_source_hash", lambda: "0" * 16)
    assert bench.traffic_from_profiles("fused_mean_kernel", "some_workload") is None
    assert bench.traffic_from_profiles("k", "old") is None


def test_hashes_of_the_kernels():
    from ddp_bucketed_gradient_amd import profiling as PF
    h = PF.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    d = PF.device_code_hash()
    if d is not None:                      # the built library's gfx950 code
        assert len(d) == 16 and d == PF.device_code_hash()
    assert PF.device_code_hash("/nonexistent/lib.so") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr
    assert r.stdout == ""


def _args(argv):
    old = sys.argv
    sys.argv = ["bench.py"] + argv
    try:
        return bench.parse()
    finally:
        sys.argv = old


@pytest.mark.parametrize("argv,name,R,cap", [
    ([], "bert_large_r8_cap25", 8, 25 << 20),
    (["--config", "2"], "resnet50_r8", 8, 25 << 20),
    (["--cap-mib", "1"], "bert_large_r8_cap1", 8, 1 << 20),
    (["--replicas", "32"], "bert_large_r32_cap25", 32, 25 << 20),
    (["--replicas", "20", "--cap-mib", "0"], "bert_large_r20_cap0", 20, 0),
    (["--config", "2", "--replicas", "16"], "resnet50_r16", 16, 25 << 20),
    (["--config", "6", "--blog-param-mib", "1", "--replicas", "8"], "blog48mib_48x1mib_r8", 8, 4 << 20),
])
def test_sync_workload_selection(argv, name, R, cap):
    """--config, --cap-mib and --replicas pick and rename the workload, so a
    stored traffic figure keyed by name never applies to another setting."""
    from workloads import configs as WC
    w = bench.sync_workload(_args(argv), WC)
    assert (w.name, w.R, w.cap_bytes) == (name, R, cap)
    assert bench.traffic_from_profiles("fused_mean_kernel", w.name) is None or name in (
        "bert_large_r8_cap25", "resnet50_r8")


def test_replicas_out_of_range_is_refused():
    from workloads import configs as WC
    for bad in ("0", "65"):
        with pytest.raises(SystemExit):
            bench.sync_workload(_args(["--replicas", bad]), WC)


def test_nosync_oracle_unit_matches_the_oracle_path():
    """The config-4 CPU baseline's unit (k micro-steps accumulated, then the
    bucketed sync, in one oracle reducer reused across units) leaves the same
    bits as a fresh oracle run, every time it runs, and counts the line's
    algorithmic bytes."""
    import numpy as np
    from oracle import reducer as OR
    from workloads import gen as WG
    numels, R, k, cap = [300, 7, 1000], 4, 3, 4 * 600
    N = sum(numels)
    steps = [[[WG.normal(WG.seed_of(4, r, v, t), n).to(__import__("torch").bfloat16)
               .view(__import__("torch").int16).numpy().view(np.uint16) for v, n in enumerate(numels)]
              for r in range(R)] for t in range(k)]
    unit = bench.nosync_oracle_unit(numels, R, k, cap, steps)
    for _ in range(2):
        assert unit() == R * N * (6 + 10 * (k - 1)) + 2 * R * 4 * N
    ref = OR.Reducer(numels, R, cap)
    acc = [[np.zeros(n, np.float32) for n in numels] for _ in range(R)]
    ref.bind(acc)
    ref.set_sync(False)
    for t in range(k):
        if t == k - 1:
            ref.set_sync(True)
        ref.no_sync_accumulate(steps[t], first=(t == 0))
    ref.sync()
    got = unit.reducer.grads                  # the unit's own accumulators
    for r in range(R):
        for v in range(len(numels)):
            assert np.array_equal(got[r][v].view(np.uint32), acc[r][v].view(np.uint32))


def test_time_oracle_threads_counts_bytes_over_time():
    calls = []

    def make(g):
        def unit():
            calls.append(g)
            return 1000
        return unit
    gbs, dt, reps = bench.time_oracle_threads(make, [0, 1, 2], 0.05)
    assert dt >= 0.05 and reps >= 1
    assert gbs == pytest.approx(1000 * (len(calls) - 3) / dt / 1e9, rel=0.05)


def test_ceiling_plan_holds_the_syncs_bytes():
    """The ceiling leg numbers each replica's copy of each variable as its own
    variable (variable-major) at R = 1 under R times the cap: the same bytes in
    about the same number of buckets as the R-replica plan."""
    from oracle import plan as OP
    from workloads import configs as WC
    for w in (WC.BERT_LARGE, WC.RESNET50):
        numels, R = w.numels(), w.R
        vm = [numels[v] for v in range(len(numels)) for _ in range(R)]
        b_sync = OP.compute_bucket_assignment_by_size(numels, 4, w.cap_bytes)
        b_ceil = OP.compute_bucket_assignment_by_size(vm, 4, R * w.cap_bytes)
        assert sum(OP.bucket_numels(b_ceil, vm)) == R * sum(numels)
        assert abs(len(b_ceil) - len(b_sync)) <= len(b_sync) // 2
        # reverse order visits the R copies of each variable together
        assert b_ceil[0][:R] == list(range(len(vm) - 1, len(vm) - 1 - R, -1))
