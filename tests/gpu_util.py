"""Helpers shared by the GPU tests: device checks, replica allocation, host
snapshots and bitwise comparison. No step of the method lives here."""
import sys

import numpy as np
import torch

import ddp_bucketed_gradient_amd as D


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device (torch.cuda.is_available() is False)")
    lib = D.lib()                      # raises ImportError if the HIP library is missing
    return lib


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def alloc_grads(numels, R, device="cuda"):
    """R x P separate fp32 tensors, the way each replica's .grad fields are
    separate allocations."""
    return [[torch.empty(n, dtype=torch.float32, device=device) for n in numels] for _ in range(R)]


def fill_from_host(grads, host):
    for row_d, row_h in zip(grads, host):
        for d, h in zip(row_d, row_h):
            d.copy_(torch.from_numpy(np.ascontiguousarray(h)))


def snapshot(grads, vs=None):
    """Host copies (float32 numpy) of grads[r][v] for every r and v in vs."""
    torch.cuda.synchronize()
    P = len(grads[0])
    vs = range(P) if vs is None else vs
    return {v: [grads[r][v].detach().cpu().numpy().copy() for r in range(len(grads))] for v in vs}


def assert_bits_equal(got, want, what=""):
    g = np.ascontiguousarray(got, dtype=np.float32).view(np.uint32)
    w = np.ascontiguousarray(want, dtype=np.float32).view(np.uint32)
    assert g.shape == w.shape, what
    gn = np.isnan(got)
    wn = np.isnan(want)
    assert np.array_equal(gn, wn), f"NaN positions differ {what}"
    diff = (g != w) & ~gn
    if diff.any():
        i = int(np.flatnonzero(diff)[0])
        raise AssertionError(f"bit mismatch {what}: {int(diff.sum())} of {g.size} elements, first at {i}: "
                             f"got {got.reshape(-1)[i]!r} ({g.reshape(-1)[i]:#010x}) "
                             f"want {want.reshape(-1)[i]!r} ({w.reshape(-1)[i]:#010x})")


def host_workers():
    """Threads for the oracle's host work (NumPy releases the GIL in its array
    operations): the process's cores, at most 16."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def closed_form_launch_log(buckets, order):
    """The launch log the in-order rule implies for a hook order: bucket b
    completes at the call c_b that marks its last member, and launches at call
    max(c_0 .. c_b) (pinned against brute force in the oracle tests)."""
    pos = {v: i for i, v in enumerate(order)}
    log, trig = [], -1
    for b, members in enumerate(buckets):
        trig = max(trig, max(pos[v] for v in members))
        log.append((b, trig))
    return log


def to_device_f32(want_host, device="cuda"):
    """Upload the oracle's expected values (host float32) once, for several
    assert_device_bits_equal calls."""
    return torch.from_numpy(np.ascontiguousarray(want_host, dtype=np.float32).reshape(-1)).to(device)


def assert_device_bits_equal(got_dev, want, what=""):
    """Bit patterns of a device tensor against the oracle's expected values
    (a host float32 array, or its upload by to_device_f32), element by element:
    compared as int32 on the device; on a mismatch the tensor is copied back and
    the first difference reported. (No NaN occurs in the full-size inputs.)"""
    want_dev = want if isinstance(want, torch.Tensor) else to_device_f32(want, got_dev.device)
    g = got_dev.reshape(-1)
    if g.numel() == want_dev.numel() and torch.equal(g.view(torch.int32), want_dev.view(torch.int32)):
        return
    assert_bits_equal(g.cpu().numpy(), want_dev.cpu().numpy(), what)
    raise AssertionError(f"device comparison failed but host comparison passed {what}")
