"""Python front end of the bucketed gradient reducer.

PyTorch supplies device memory and streams; every step of the path runs in the
native library (``include/ddpb.h``). The class keeps references to the tensors
and streams it was bound to, so the caching allocator cannot hand their memory
out while side-stream kernels still use it.
"""
from __future__ import annotations

import sys as _sys
from typing import List, Optional, Sequence

from . import _abi
from ._abi import (BF16, F32, MODE_FUSED, MODE_STAGED, BIND_DEVICE_TIMESTAMPS, BIND_TIME_LAUNCHES,  # noqa: F401
                   BIND_ROCTX, BIND_OVERLAP)

MiB = 1 << 20


class StepTable:
    """Checked, marshalled addresses of one R x P set of step gradients
    (Reducer.step_table). It holds references to the tensors, which must
    keep their storage (no resize or set_) while the table is in use."""
    __slots__ = ("ptrs", "code", "tensors")

    def __init__(self, ptrs, code: int, tensors):
        self.ptrs, self.code, self.tensors = ptrs, code, tensors


class Reducer:
    def __init__(self, shapes: Sequence[Sequence[int]], R: int, bucket_cap_bytes: int = 25 * MiB,
                 lib: Optional[_abi.Lib] = None):
        self.lib = lib if lib is not None else _abi.lib()
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        self.P = len(self.shapes)
        self.R = int(R)
        self.cap = int(bucket_cap_bytes)
        self._numel = []
        for s in self.shapes:
            n = 1
            for d in s:
                n *= d
            self._numel.append(n)
        self.h = self.lib.reducer_create(self.shapes, F32, self.cap, self.R)
        self._keep = []

    # -- plan queries -------------------------------------------------------------
    @property
    def num_buckets(self) -> int:
        return self.lib.num_buckets(self.h)

    def buckets(self) -> List[List[int]]:
        return [self.lib.get_bucket(self.h, b)[0] for b in range(self.num_buckets)]

    def bucket_bytes(self) -> List[int]:
        return [self.lib.get_bucket(self.h, b)[1] for b in range(self.num_buckets)]

    def locator(self, v: int):
        return self.lib.get_locator(self.h, v)

    def workspace_bytes(self, mode: int = MODE_FUSED) -> int:
        return self.lib.workspace_bytes(self.h, mode)

    # -- binding -------------------------------------------------------------------
    def bind(self, grads, compute_stream=None, side_streams=None, mode: int = MODE_FUSED, flags: int = 0):
        """grads[r][v]: contiguous fp32 CUDA tensor with the v-th shape's numel."""
        import torch
        if len(grads) != self.R or any(len(row) != self.P for row in grads):
            raise ValueError("grads must be R x P")
        dev = None
        ptrs = []
        for r in range(self.R):
            for v in range(self.P):
                t = grads[r][v]
                n = self._numel[v]
                if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or t.numel() != n:
                    raise ValueError(f"grads[{r}][{v}] must be a contiguous fp32 CUDA tensor of {n} elements")
                dev = t.device if dev is None else dev
                ptrs.append(t.data_ptr())
        if dev is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        compute = compute_stream if compute_stream is not None else torch.cuda.current_stream(dev)
        # default: two side streams, buckets alternate between them so that
        # consecutive bucket kernels overlap each other's start-up and drain
        sides = list(side_streams) if side_streams else [torch.cuda.Stream(device=dev) for _ in range(2)]
        nbytes = self.lib.workspace_bytes(self.h, mode)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
        self._keep = [grads, ws, compute, sides]
        self.compute_stream, self.side_streams, self.workspace = compute, sides, ws
        self.lib.bind(self.h, ptrs, ws.data_ptr() if ws is not None else 0, nbytes, compute.cuda_stream,
                      [s.cuda_stream for s in sides], mode, flags)

    def bind_static(self, grads, compute_stream=None, mode: int = MODE_FUSED):
        """Allocation-free binding (ddpb_bind_static): the library's tables sit
        in its static device array and the reductions run on the compute
        stream; grads as for bind."""
        import torch
        if len(grads) != self.R or any(len(row) != self.P for row in grads):
            raise ValueError("grads must be R x P")
        ptrs = []
        for r in range(self.R):
            for v in range(self.P):
                t = grads[r][v]
                n = self._numel[v]
                if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or t.numel() != n:
                    raise ValueError(f"grads[{r}][{v}] must be a contiguous fp32 CUDA tensor of {n} elements")
                ptrs.append(t.data_ptr())
        compute = compute_stream if compute_stream is not None else torch.cuda.current_stream()
        self._keep = [grads, compute]
        self.compute_stream, self.side_streams, self.workspace = compute, [compute], None
        self.lib.bind_static(self.h, ptrs, compute.cuda_stream, mode)

    def bind_bucket_views(self, device=None, compute_stream=None, side_streams=None, flags: int = 0):
        """gradient_as_bucket_view: allocate one flat fp32 storage per replica
        in bucket layout (all R in one allocation), bind them, and return R x P
        gradient views into them
        (shaped like the parameters). Write each replica's gradients into its
        views; the reduction averages them in place."""
        import torch
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        n = self.lib.view_storage_elems(self.h)
        # One allocation holds every replica's storage, replica r at r * stride
        # elements (4 KiB between storages, 256-byte aligned): the in-place
        # reduction streamed 0.5-2 % faster over this placement than over R
        # separate allocations (BERT-large, R = 8: 5,694-5,700 against
        # 5,584-5,652 GB/s, three rounds on one box).
        stride = (max(n, 1) + 1024 + 63) // 64 * 64
        flat = torch.zeros(self.R * stride, dtype=torch.float32, device=dev)
        stores = [flat[r * stride:r * stride + max(n, 1)] for r in range(self.R)]
        views = []
        for r in range(self.R):
            row = []
            for v, shape in enumerate(self.shapes):
                off = self.lib.get_view_offset(self.h, v)
                numel = 1
                for d in shape:
                    numel *= d
                row.append(stores[r][off:off + numel].view(shape))
            views.append(row)
        compute = compute_stream if compute_stream is not None else torch.cuda.current_stream(dev)
        sides = list(side_streams) if side_streams else [torch.cuda.Stream(device=dev) for _ in range(2)]
        self._keep = [flat, stores, views, compute, sides]
        self.compute_stream, self.side_streams, self.workspace = compute, sides, None
        self.lib.bind_bucket_views(self.h, [s.data_ptr() for s in stores], n, compute.cuda_stream,
                                   [s.cuda_stream for s in sides], flags)
        return views

    def rebuild_buckets(self, bucket_cap_bytes: Optional[int] = None):
        """Re-plan the buckets from the last finished iteration's hook order.
        The reducer must be bound again afterwards (``bind`` or
        ``bind_bucket_views``; views change)."""
        cap = self.cap if bucket_cap_bytes is None else int(bucket_cap_bytes)
        self.lib.rebuild_buckets(self.h, cap)
        self.cap = cap

    def ready_order(self) -> List[int]:
        return self.lib.get_ready_order(self.h)

    def view_offset(self, v: int) -> int:
        return self.lib.get_view_offset(self.h, v)

    def bind_ptrs(self, ptrs: Sequence[int], workspace: int = 0, ws_bytes: int = 0, compute_stream: int = 0,
                  side_streams: Sequence[int] = (0,), mode: int = MODE_FUSED, flags: int = 0):
        """Raw-pointer bind (used by the host-only tests)."""
        self.lib.bind(self.h, ptrs, workspace, ws_bytes, compute_stream, side_streams, mode, flags)

    # -- iteration -------------------------------------------------------------------
    def ensure_prior_reduction_finished(self):
        self.lib.ensure_prior_reduction_finished(self.h)

    def mark_ready(self, v: int):
        self.lib.mark_ready(self.h, v)

    def mark_ready_many(self, vs: Sequence[int]):
        self.lib.mark_ready_many(self.h, vs)

    def finalize(self):
        self.lib.finalize(self.h)

    def set_sync(self, enabled: bool):
        self.lib.set_sync(self.h, enabled)

    def reset(self):
        self.lib.reset(self.h)

    def sync(self, order: Optional[Sequence[int]] = None):
        """One synchronisation: every hook in ``order`` (default: last-defined
        parameter first), then finalize."""
        if order is None:
            order = range(self.P - 1, -1, -1)
        mr = self.lib.mark_ready
        h = self.h
        for v in order:
            mr(h, v)
        self.lib.finalize(h)

    def no_sync_accumulate(self, steps, first_step: bool):
        """steps[r][v]: contiguous fp32 or bf16 CUDA tensor per replica/variable,
        or None where that replica produced no gradient (zeros on the first
        step, unchanged afterwards); or a StepTable made by step_table()."""
        t = steps if isinstance(steps, StepTable) else self.step_table(steps)
        self.lib.no_sync_accumulate(self.h, t.ptrs, t.code, first_step)

    def set_sync_step(self, steps, first_step: bool = False):
        """The last local step of a no_sync run, added to the gradients by the
        coming synchronisation itself (set before its first hook; the same
        result as no_sync_accumulate followed by the sync, in one pass).
        ``steps`` as for no_sync_accumulate; the tensors must stay alive until
        finalize."""
        t = steps if isinstance(steps, StepTable) else self.step_table(steps)
        self.lib.set_sync_step(self.h, t.ptrs, t.code, first_step)
        self._keep_steps = t

    def step_table(self, steps) -> "StepTable":
        """Check an R x P set of step gradients once and marshal their
        addresses, for callers that pass the same tensors to several
        no_sync_accumulate / set_sync_step calls (the checks and the pointer
        array cost about 2 ms of host time for 3,000 tensors)."""
        import torch
        if len(steps) != self.R or any(len(row) != self.P for row in steps):
            raise ValueError("steps must be R x P")
        present = [t for row in steps for t in row if t is not None]
        dt = present[0].dtype if present else torch.float32
        code = {torch.float32: F32, torch.bfloat16: BF16}.get(dt)
        if code is None:
            raise ValueError("step gradients must be fp32 or bf16")
        numel = self._numel
        ptrs = []
        append = ptrs.append
        for r, row in enumerate(steps):
            for v, t in enumerate(row):
                if t is None:
                    append(0)
                    continue
                if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                    raise ValueError("step gradients must be contiguous CUDA tensors of one dtype")
                if t.numel() != numel[v]:
                    raise ValueError(f"steps[{r}][{v}] has {t.numel()} elements, the variable {numel[v]}")
                append(t.data_ptr())
        return StepTable(_abi.ptr_array(ptrs), code, steps)

    def set_local_used(self, used):
        """Which replicas use which variables in the coming backward pass: an
        R x P array-like of booleans (or None for all used). Calls before one
        synchronisation OR together."""
        if used is None:
            self.lib.set_local_used(self.h, None)
            return
        import numpy as np
        u = np.asarray(used, dtype=bool)
        if u.shape != (self.R, self.P):
            raise ValueError(f"used flags must have shape ({self.R}, {self.P})")
        self.lib.set_local_used(self.h, np.ascontiguousarray(u, dtype=np.uint8).ravel())

    # -- diagnostics -------------------------------------------------------------------
    def launch_log(self, with_stamps: bool = False):
        return self.lib.get_launch_log(self.h, with_stamps)

    def launch_times_ms(self, iterations_ago: int = 0, with_starts: bool = False):
        return self.lib.get_launch_times(self.h, iterations_ago, with_starts)

    def set_launch_blocks(self, max_blocks: int):
        """Cap the workgroups per reduction launch (0 = whole GPU)."""
        self.lib.set_launch_blocks(self.h, max_blocks)

    def set_workgroups_per_cu(self, n: int):
        """At most n (1 or 2) reduction workgroups per compute unit; 0 = no
        limit (denser sharing with concurrent backward kernels)."""
        self.lib.set_workgroups_per_cu(self.h, n)

    def device_clock_hz(self) -> int:
        return self.lib.device_clock_hz(self.h)

    def close(self):
        if self.h:
            self.lib.destroy(self.h)
            self.h = None
            self._keep = []
            self._keep_steps = None

    def __del__(self):
        try:
            if _sys.is_finalizing():     # the HIP runtime may already be gone
                return
            self.close()
        except BaseException:
            pass
