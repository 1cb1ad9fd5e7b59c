"""The nn.Linear(10, 10) example in closed form (oracle).

From [TP] "Example": each of two ranks wraps nn.Linear(10, 10), feeds a
20 x 10 batch, takes loss = mean(outputs ** 2), runs backward and one SGD step
with lr = 0.001; the constructor broadcasts rank 0's parameters, and after
backward every rank holds the mean of the ranks' local gradients, so the
replicas stay identical.

With y = x W^T + b (20 x 10) and L = (1/200) * sum(y**2):
    dL/dy = y / 100,   dW = (1/100) y^T x,   db = (1/100) sum_n y[n, :].
The per-rank gradients are computed in float64 from the float32 inputs and
rounded once to float32.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np


def forward(x: np.ndarray, W: np.ndarray, b: np.ndarray) -> np.ndarray:
    x64, W64, b64 = (np.asarray(a, dtype=np.float64) for a in (x, W, b))
    return x64 @ W64.T + b64


def grads(x: np.ndarray, W: np.ndarray, b: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(dW [10,10], db [10]) of mean(y**2), float64 math, float32 result."""
    y = forward(x, W, b)
    n_out = y.size                     # the mean runs over every output element
    gy = y * (2.0 / n_out)
    dW = gy.T @ np.asarray(x, dtype=np.float64)
    db = gy.sum(axis=0)
    return dW.astype(np.float32), db.astype(np.float32)


def loss(x: np.ndarray, W: np.ndarray, b: np.ndarray) -> float:
    y = forward(x, W, b)
    return float((y ** 2).mean())


def broadcast_from_rank0(params: List[List[np.ndarray]]) -> List[List[np.ndarray]]:
    """Every rank takes rank 0's parameters ([TP] "Internal Design",
    construction; [PDTI] §2)."""
    src = params[0]
    return [[np.array(p, copy=True) for p in src] for _ in params]


def sgd_step(params: List[np.ndarray], grads_: List[np.ndarray], lr: float) -> List[np.ndarray]:
    """p <- p - lr * g in float32 (plain SGD, no momentum)."""
    lr32 = np.float32(lr)
    return [(p - lr32 * g).astype(np.float32) for p, g in zip(params, grads_)]
