"""Pins for the float64 softmax -> TopK oracle (oracle/topk.py).

A slip (TopK on the wrong axis, ascending order, ties to the higher index,
a missing max shift or normaliser, a dropped rescale in the incremental
merge) fails at least one of:
  * a pure-Python version (math.exp, math.fsum, sorted with key (-x, index));
  * torch in float64: softmax, then a stable descending sort;
  * closed forms: equal logits give p = 1/E and indices 0..k-1; one dominant
    logit takes almost all the mass;
  * invariants: the top-E values sum to 1; adding a constant to a row changes
    nothing; incremental == three-pass for any chunking and chunk order.
"""
import math

import numpy as np
import pytest
import torch

from oracle.topk import softmax_topk, softmax_topk_incremental


def logits(rows, E, seed, ties=False):
    x = np.random.default_rng(seed).standard_normal((rows, E)) * 2.0
    if ties:
        x = np.round(x * 4) / 4  # many equal values
    return x


@pytest.mark.parametrize("E,k,ties", [(5, 2, False), (16, 4, True), (33, 33, False), (256, 8, True)])
def test_matches_pure_python(E, k, ties):
    x = logits(6, E, E + k, ties)
    vals, idx = softmax_topk(x, k)
    for r in range(6):
        m = max(x[r])
        ex = [math.exp(v - m) for v in x[r]]
        z = math.fsum(ex)
        best = sorted(range(E), key=lambda e: (-x[r][e], e))[:k]
        assert list(idx[r]) == best
        for j, e in enumerate(best):
            assert abs(vals[r, j] - ex[e] / z) <= 1e-15


@pytest.mark.parametrize("ties", [False, True])
def test_matches_torch_stable_sort(ties):
    x = logits(40, 128, 3, ties)
    vals, idx = softmax_topk(x, 10)
    t = torch.tensor(x)
    p = torch.softmax(t, dim=1)
    order = torch.sort(-t, dim=1, stable=True).indices[:, :10]
    np.testing.assert_array_equal(idx, order.numpy())
    np.testing.assert_allclose(vals, torch.gather(p, 1, order).numpy(), rtol=1e-13)


def test_closed_forms():
    vals, idx = softmax_topk(np.zeros((2, 10)), 4)
    np.testing.assert_array_equal(idx, [[0, 1, 2, 3]] * 2)
    np.testing.assert_allclose(vals, 0.1, rtol=1e-15)
    x = np.zeros((1, 8))
    x[0, 5] = 50.0
    vals, idx = softmax_topk(x, 2)
    assert idx[0, 0] == 5 and idx[0, 1] == 0
    z = 1 + 7 * math.exp(-50)
    assert vals[0, 0] == pytest.approx(1 / z, rel=1e-15) and vals[0, 1] == pytest.approx(math.exp(-50) / z, rel=1e-13)


def test_invariants():
    x = logits(9, 64, 4)
    vals, idx = softmax_topk(x, 64)
    np.testing.assert_allclose(vals.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(np.diff(vals, axis=1) <= 0)
    v2, i2 = softmax_topk(x + 7.5, 64)
    np.testing.assert_array_equal(i2, idx)
    np.testing.assert_allclose(v2, vals, rtol=1e-13)


@pytest.mark.parametrize("chunk", [1, 7, 64, 256])
@pytest.mark.parametrize("ties", [False, True])
def test_incremental_equals_three_pass(chunk, ties):
    x = logits(12, 256, 5, ties) * 10  # wide spread: the rescale matters
    vals, idx = softmax_topk(x, 8)
    vi, ii = softmax_topk_incremental(x, 8, chunk)
    np.testing.assert_array_equal(ii, idx)
    np.testing.assert_allclose(vi, vals, rtol=1e-12)


def test_incremental_is_order_independent():
    x = logits(5, 200, 6, ties=True)
    vals, idx = softmax_topk(x, 16)
    for seed in range(3):
        order = np.random.default_rng(seed).permutation(-(-200 // 16))
        vi, ii = softmax_topk_incremental(x, 16, 16, order=order)
        np.testing.assert_array_equal(ii, idx)
        np.testing.assert_allclose(vi, vals, rtol=1e-12)
