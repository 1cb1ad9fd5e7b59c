"""Reducer state machine and bucket reduction (oracle).

R data-parallel replicas are held side by side: ``grads[r][v]`` is replica r's
gradient of variable v, a 1-D float32 NumPy array that the reducer updates in
place, as the real reducer writes the averaged values back into every
parameter's ``.grad``.

Steps, in the pages' order:

* per-bucket state: a pending count equal to the number of member variables
  ([Li] "Overlapping Computation with Communication", per-hook logic;
  [C30] "Variable 到 Bucket");
* ``mark_ready(v)``: copy v's gradient into its narrowed view of the flat
  bucket, decrement pending; when it reaches zero the bucket is ready
  ([Li] same subsection; [PDTI] §2);
* ready buckets are launched strictly in bucket-index order; a bucket that
  becomes ready before its predecessors were launched waits (is parked) and is
  launched as soon as every earlier bucket has been ([Li] "Launching AllReduce
  in order"; [C30] "Bucket 必须按序发起");
* a launched bucket is averaged over the replicas and the result is written
  back to each member's gradient on every replica ([TP] "Internal Design",
  backward pass; [PDTI] §3; [Li] "After AllReduce: writing averaged gradients
  back");
* ``finalize()`` at the end of backward requires every bucket to have been
  launched; otherwise the reduction is incomplete and the next iteration fails
  ([TP] "When a parameter never receives a gradient"; [C30] "未检测的失败");
* ``no_sync``: while synchronisation is off the hooks do nothing and gradients
  accumulate additively across backward passes ([Li] "Gradient Accumulation
  (no_sync)"; [TP] "Gradient sync you can turn off").

Readings of points the pages leave open:
* the average is the sum over replicas 0..R-1 taken left to right in float32
  (acc = g_0, then acc + g_1, ...), followed by one IEEE division by R
  (round to nearest even, subnormals kept). For float32 the pages say the
  bucket is averaged directly; dividing first and summing after would give the
  same bits for power-of-two R in the absence of underflow, but not in general;
* copy-back happens per bucket right after its reduction; ``finalize`` only
  checks completeness and resets the per-iteration state;
* all R replicas run their hooks in lockstep: one ``mark_ready(v)`` means v's
  gradient is final on every replica;
* marking the same variable twice in one iteration is an error.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

from .plan import compute_bucket_assignment_by_size, locators, bucket_numels


class ReductionIncomplete(RuntimeError):
    """The prior iteration did not finish reducing every bucket."""


class DoubleReady(RuntimeError):
    """A variable was marked ready twice in one iteration."""


def fixed_order_mean(bufs: Sequence[np.ndarray]) -> np.ndarray:
    """m = fl(fl(... fl(g_0 + g_1) ... + g_{R-1}) / R), elementwise, float32."""
    R = len(bufs)
    if R < 1:
        raise ValueError("need at least one replica")
    acc = np.array(bufs[0], dtype=np.float32, copy=True)
    for r in range(1, R):
        acc = acc + np.asarray(bufs[r], dtype=np.float32)
    return acc / np.float32(R)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 (given as uint16 bit patterns) to float32 exactly: a bf16
    value is the upper half of the binary32 encoding."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


class Reducer:
    """``gradient_as_bucket_view=True`` follows [TP] "Internal Design"
    (backward pass) and [C30] section "gradient_as_bucket_view": each
    parameter's gradient *is* its narrowed view of the flat bucket, so the
    hook copies nothing and the averaged bucket is the averaged gradient. The
    views are handed out by :meth:`views` and the caller writes gradients
    into them."""

    def __init__(self, numels: Sequence[int], R: int, bucket_cap_bytes: int,
                 elem_size: int = 4, gradient_as_bucket_view: bool = False):
        if R < 1:
            raise ValueError("R must be >= 1")
        self.numels = [int(n) for n in numels]
        self.P = len(self.numels)
        self.R = R
        self.elem_size = elem_size
        self.cap = bucket_cap_bytes
        self.sync_enabled = True
        self.failed = False
        self.grads: Optional[List[List[np.ndarray]]] = None
        self.launch_log: List[Tuple[int, int]] = []   # (bucket, index of triggering mark_ready call)
        self.as_view = bool(gradient_as_bucket_view)
        self.order_now: List[int] = []                # hooks of the current iteration, in order
        self.last_ready_order: Optional[List[int]] = None
        self.used_acc: Optional[np.ndarray] = None    # R x P used flags, OR-ed over no_sync steps
        self._plan(compute_bucket_assignment_by_size(self.numels, elem_size, bucket_cap_bytes))
        self._reset_iteration()

    def _plan(self, buckets: List[List[int]]):
        self.buckets = buckets
        self.loc = locators(self.buckets, self.numels)
        self.B = len(self.buckets)
        self.bucket_elems = bucket_numels(self.buckets, self.numels)
        # per-replica flat buckets (the pages' flat bucket buffers)
        self.flat = [[np.zeros(n, dtype=np.float32) for n in self.bucket_elems] for _ in range(self.R)]
        self.averaged = [np.zeros(n, dtype=np.float32) for n in self.bucket_elems]
        if self.as_view:
            self.grads = [[self.flat[r][L.bucket][L.offset:L.offset + L.length] for L in self.loc]
                          for r in range(self.R)]

    def rebuild_buckets(self, bucket_cap_bytes: Optional[int] = None) -> bool:
        """Re-plan from the order in which the hooks fired in the last finished
        iteration ([C30] "第一次迭代为何不同"): the rebuild needs the prior
        reduction to be complete, then packs the parameters in their ready
        order with the same cap rule. Returns False when no finished iteration
        was recorded. In bucket-view mode the views are new (re-fetch them)."""
        if self.failed or self.started:
            raise ReductionIncomplete("rebuild needs the prior iteration to have finished reducing")
        if self.last_ready_order is None:
            return False
        if bucket_cap_bytes is not None:
            self.cap = bucket_cap_bytes
        self._plan(compute_bucket_assignment_by_size(self.numels, self.elem_size, self.cap,
                                                     order=self.last_ready_order))
        self._reset_iteration()              # copying mode: the caller's gradients stay bound
        return True

    def views(self) -> List[List[np.ndarray]]:
        """R x P gradient views into the flat buckets (bucket-view mode only)."""
        if not self.as_view:
            raise RuntimeError("views exist only with gradient_as_bucket_view=True")
        return self.grads

    # -- state ---------------------------------------------------------------
    def _reset_iteration(self):
        self.pending = [len(m) for m in self.buckets]
        self.ready = [False] * self.P
        self.next_bucket = 0
        self.calls = 0
        self.started = False             # the iteration's first hook has run
        self.order_now = []

    def bind(self, grads: List[List[np.ndarray]]):
        if self.as_view:
            raise RuntimeError("in bucket-view mode the gradients are the views; use views()")
        if len(grads) != self.R or any(len(row) != self.P for row in grads):
            raise ValueError("grads must be R x P")
        for row in grads:
            for v, g in enumerate(row):
                if g.dtype != np.float32 or g.ndim != 1 or g.size != self.numels[v]:
                    raise ValueError(f"grad {v}: need flat float32 of {self.numels[v]} elements")
        self.grads = grads

    def set_sync(self, enabled: bool):
        if self.started:
            raise RuntimeError("cannot toggle sync in the middle of an iteration")
        self.sync_enabled = bool(enabled)

    def ensure_prior_reduction_finished(self):
        if self.failed or self.started:
            self.failed = True
            raise ReductionIncomplete(
                "prior iteration did not finish reducing every bucket")

    # -- hooks ---------------------------------------------------------------
    # -- unused parameters ---------------------------------------------------
    def set_local_used(self, used):
        """Which replicas used which variables in the coming backward pass
        (R x P booleans), as the forward's graph walk would find them ([Li]
        "Handling Unused Parameters"; [TP] forward pass with
        find_unused_parameters). Under no_sync the flags of successive calls
        are OR-ed together and serve the next synchronisation ([Li] "Gradient
        Accumulation (no_sync)"). Without any call every variable is used."""
        if self.started:
            raise RuntimeError("set_local_used must come before the iteration's hooks")
        u = np.asarray(used, dtype=bool).reshape(self.R, self.P)
        self.used_acc = u.copy() if self.used_acc is None else (self.used_acc | u)

    def globally_used(self) -> np.ndarray:
        """The OR over replicas of the used flags (the bitmap all-reduce)."""
        if self.used_acc is None:
            return np.ones(self.P, dtype=bool)
        return self.used_acc.any(axis=0)

    def _zero_slices(self, r: int, v: int):
        L = self.loc[v]
        self.flat[r][L.bucket][L.offset:L.offset + L.length] = 0.0

    def _mark_unused_ready(self, call: int):
        """At the iteration's first hook: zero the bucket slices of variables a
        replica did not use, and treat globally unused variables as ready."""
        if self.used_acc is None:
            return
        G = self.globally_used()
        for r in range(self.R):
            for v in range(self.P):
                if not self.used_acc[r, v]:
                    self._zero_slices(r, v)
        for v in range(self.P):
            if not G[v]:
                self.ready[v] = True
                b = self.loc[v].bucket
                self.pending[b] -= 1
                if self.pending[b] == 0:
                    self._mark_bucket_ready(b, call)

    # -- hooks ---------------------------------------------------------------
    def mark_ready(self, v: int):
        if not (0 <= v < self.P):
            raise IndexError(v)
        if not self.sync_enabled:
            return
        if self.failed:
            raise ReductionIncomplete("prior iteration did not finish reducing every bucket")
        call = self.calls
        if not self.started:
            # [C30] "Unused Parameter": unused variables are marked ready once
            # per iteration, when its first hook runs (even if that hook then
            # fails), never again within the iteration.
            self.started = True
            self._mark_unused_ready(call)
        if self.ready[v]:
            raise DoubleReady(v)
        self.ready[v] = True
        self.order_now.append(v)
        self.calls += 1
        L = self.loc[v]
        if not self.as_view:             # the view copy: bucket.narrow(offset, numel) <- grad
            for r in range(self.R):
                if self.used_acc is not None and not self.used_acc[r, v]:
                    self._zero_slices(r, v)  # a replica without this gradient contributes zeros
                else:
                    self.flat[r][L.bucket][L.offset:L.offset + L.length] = self.grads[r][v]
        self.pending[L.bucket] -= 1
        if self.pending[L.bucket] == 0:
            self._mark_bucket_ready(L.bucket, call)

    def _mark_bucket_ready(self, b: int, call: int):
        if b > self.next_bucket:
            return                        # parked until every earlier bucket launched
        while self.next_bucket < self.B and self.pending[self.next_bucket] == 0:
            self._launch(self.next_bucket, call)
            self.next_bucket += 1

    def _launch(self, b: int, call: int):
        m = fixed_order_mean([self.flat[r][b] for r in range(self.R)])
        self.averaged[b] = m
        if self.as_view:                 # the bucket is the gradient storage
            for r in range(self.R):
                self.flat[r][b][...] = m
        else:
            G = self.globally_used()
            for v in self.buckets[b]:
                if not G[v]:
                    continue             # globally unused: its gradients are left untouched
                L = self.loc[v]
                for r in range(self.R):
                    self.grads[r][v][...] = m[L.offset:L.offset + L.length]
        self.launch_log.append((b, call))

    def finalize(self):
        if not self.sync_enabled and not self.started:
            return
        if self.failed:                  # latched until reset, like the hooks
            raise ReductionIncomplete("prior iteration did not finish reducing every bucket")
        if not self.started:             # no hook fired: only unused variables, if any
            self.started = True
            self._mark_unused_ready(0)
        if self.next_bucket != self.B:
            self.failed = True
            raise ReductionIncomplete(
                f"only {self.next_bucket} of {self.B} buckets were reduced")
        # a rebuild needs every variable's place in the ready order; an
        # iteration with unused variables does not give one
        self.last_ready_order = list(self.order_now) if len(self.order_now) == self.P else None
        self.used_acc = None             # the flags served this synchronisation
        self._reset_iteration()

    def reset(self):
        """Recovery after a failed iteration (the failure itself surfaces at
        the next forward, [TP] "When a parameter never receives a gradient").
        The used flags served the synchronisation that failed and are dropped
        with it: they serve one synchronising iteration ([Li] "Gradient
        Accumulation (no_sync)")."""
        self.failed = False
        self.used_acc = None
        self._reset_iteration()

    # -- no_sync -------------------------------------------------------------
    def no_sync_accumulate(self, step: List[List[np.ndarray]], first: bool):
        """One local backward's contribution: ``grad = step`` on the first
        micro-step, ``grad += step`` afterwards (float32). ``step`` holds
        float32 arrays, or uint16 arrays of bf16 bit patterns; ``None`` means
        that replica produced no gradient for that variable (it contributes
        zeros).

        A local backward belongs between iterations: inside an open iteration
        (its first hook ran, finalize did not) it is refused, and so it is
        while a failed iteration is latched ([TP] "When a parameter never
        receives a gradient": the next iteration cannot start)."""
        if self.failed:
            raise ReductionIncomplete("prior iteration did not finish reducing every bucket")
        if self.started:
            raise RuntimeError("no_sync_accumulate: an iteration is in progress")
        for r in range(self.R):
            for v in range(self.P):
                s = step[r][v]
                if s is None:
                    if first:
                        self.grads[r][v][...] = 0.0
                    continue
                s32 = bf16_bits_to_f32(s) if s.dtype == np.uint16 else np.asarray(s, dtype=np.float32)
                if first:
                    self.grads[r][v][...] = s32
                else:
                    self.grads[r][v][...] = self.grads[r][v] + s32

    # -- one whole synchronisation -------------------------------------------
    def sync(self, order: Optional[Sequence[int]] = None):
        """Run every hook in ``order`` (default: reverse index) and finalize."""
        if order is None:
            order = range(self.P - 1, -1, -1)
        for v in order:
            self.mark_ready(v)
        self.finalize()
