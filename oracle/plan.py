"""Bucket assignment and the variable locator (oracle).

Rule, from [Li] "Gradient Bucketing" (paper §3.2.2), [TP] "Internal Design"
(construction) and [C30] "bucket_cap_mb 不是张量切分器":

* parameters are visited in reverse ``Model.parameters()`` order;
* each whole tensor is appended to the open bucket and its byte size added;
* once the bucket's size reaches or exceeds the cap the bucket is closed
  (so one tensor larger than the cap still forms a single, larger bucket);
* a tensor is never split between buckets.

Readings where the pages leave a step open:
* the comparison is ``>=`` ("reaches or exceeds"); a cap of 0 therefore puts
  every tensor in its own bucket, the pages' "0 MB" per-gradient case;
* a final, partly filled bucket is emitted last (every parameter belongs to
  exactly one bucket);
* inside a bucket, tensors sit back to back in insertion order with no padding
  (each parameter owns a narrowed view ``[offset, offset + numel)``).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence


def compute_bucket_assignment_by_size(numels: Sequence[int], elem_size: int,
                                      cap_bytes: int, order: Sequence[int] = None) -> List[List[int]]:
    """Return the buckets as lists of variable indices, bucket 0 first.

    ``order`` is the visiting order: by default the reverse of the definition
    order; a bucket rebuild passes the order in which the gradients became
    ready in a finished iteration ([C30] "第一次迭代为何不同": the rebuilt
    parameters are packed in their actual ready order with the same rule)."""
    if order is None:
        order = range(len(numels) - 1, -1, -1)
    elif sorted(order) != list(range(len(numels))):
        raise ValueError("order must be a permutation of the variable indices")
    buckets: List[List[int]] = []
    current: List[int] = []
    size = 0
    for v in order:
        current.append(v)
        size += int(numels[v]) * int(elem_size)
        if size >= cap_bytes:
            buckets.append(current)
            current = []
            size = 0
    if current:
        buckets.append(current)
    return buckets


@dataclass(frozen=True)
class Locator:
    """variable_index -> (bucket_index, intra_bucket_index, offset, length);
    offset and length are in elements of the flat bucket ([C30] "Variable 到
    Bucket")."""
    bucket: int
    intra: int
    offset: int
    length: int


def locators(buckets: List[List[int]], numels: Sequence[int]) -> List[Locator]:
    out: List[Locator] = [None] * len(numels)  # type: ignore[list-item]
    for b, members in enumerate(buckets):
        off = 0
        for i, v in enumerate(members):
            out[v] = Locator(b, i, off, int(numels[v]))
            off += int(numels[v])
    return out


def bucket_numels(buckets: List[List[int]], numels: Sequence[int]) -> List[int]:
    return [sum(int(numels[v]) for v in members) for members in buckets]
