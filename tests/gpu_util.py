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
