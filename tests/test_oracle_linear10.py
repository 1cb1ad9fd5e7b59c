"""Pins for the nn.Linear(10, 10) example: closed-form gradients against
autograd, the rank-0 broadcast, and replica equality after one step."""
import numpy as np
import torch

from conftest import load_golden
from oracle import linear10 as OL
from oracle import reducer as OR
from workloads import gen as WG


def _autograd_grads(x, W, b):
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    out = torch.tensor(x, dtype=torch.float64) @ Wt.T + bt
    out.square().mean().backward()
    return Wt.grad.numpy(), bt.grad.numpy()


def test_closed_form_matches_autograd():
    g = load_golden("tp_linear10_example.json")
    W, b = (t.numpy() for t in WG.linear10_init(0))
    for r in range(g["world_size"]):
        x = WG.linear10_batch(r).numpy()
        assert x.shape == tuple(g["batch"])
        dW, db = OL.grads(x, W, b)
        aW, ab = _autograd_grads(x, W, b)
        # the oracle rounds its float64 result once to float32
        assert np.allclose(dW.astype(np.float64), aW, rtol=2 ** -23, atol=0)
        assert np.allclose(db.astype(np.float64), ab, rtol=2 ** -23, atol=0)


def _mutants():
    def halved(x, W, b):                    # dropped the factor 2 of d(y^2)
        y = OL.forward(x, W, b)
        return ((y / 200).T @ x).astype(np.float32), (y / 200).sum(0).astype(np.float32)

    def transposed(x, W, b):                # dW transposed
        y = OL.forward(x, W, b)
        return (x.T @ (y / 100)).astype(np.float32), (y / 100).sum(0).astype(np.float32)

    def wrong_rows(x, W, b):                # rows of y paired with the wrong inputs
        y = OL.forward(x, W, b)
        return ((y / 100).T @ x[::-1]).astype(np.float32), (y / 100).sum(0).astype(np.float32)

    def bias_sign(x, W, b):
        y = OL.forward(x, W, b)
        return ((y / 100).T @ x).astype(np.float32), (-(y / 100).sum(0)).astype(np.float32)
    return [halved, transposed, wrong_rows, bias_sign]


def test_closed_form_planted_mistakes_are_caught(monkeypatch):
    import pytest
    for m in _mutants():
        monkeypatch.setattr(OL, "grads", m)
        with pytest.raises(AssertionError):
            test_closed_form_matches_autograd()


def test_broadcast_then_one_step_keeps_replicas_identical():
    g = load_golden("tp_linear10_example.json")
    R = g["world_size"]
    inits = [[t.numpy() for t in WG.linear10_init(r)] for r in range(R)]
    assert not np.array_equal(inits[0][0], inits[1][0])          # seeded differently
    params = OL.broadcast_from_rank0(inits)
    for r in range(R):
        for p, p0 in zip(params[r], inits[0]):
            assert np.array_equal(p, p0)
    # per-rank local gradients, in Model.parameters() order [weight, bias]
    local = []
    for r in range(R):
        dW, db = OL.grads(WG.linear10_batch(r).numpy(), *params[r])
        local.append([dW.reshape(-1).copy(), db.copy()])
    grads = [[a.copy() for a in row] for row in local]
    red = OR.Reducer([100, 10], R, 25 << 20)
    assert red.buckets == [[1, 0]]
    red.bind(grads)
    red.sync()
    for v in range(2):
        want = OR.fixed_order_mean([local[r][v] for r in range(R)])
        for r in range(R):
            assert np.array_equal(grads[r][v], want)
    # the averaged gradient differs from every local one (the data differ)
    assert not np.array_equal(grads[0][0], local[0][0])
    new = [OL.sgd_step(params[r], [grads[r][0].reshape(10, 10), grads[r][1]], g["lr"]) for r in range(R)]
    for r in range(1, R):
        for p, q in zip(new[r], new[0]):
            assert np.array_equal(p, q)
    # the step lowers the loss averaged over the ranks' batches
    before = np.mean([OL.loss(WG.linear10_batch(r).numpy(), *params[r]) for r in range(R)])
    after = np.mean([OL.loss(WG.linear10_batch(r).numpy(), *new[r]) for r in range(R)])
    assert after < before
