"""Pins for the float64 LayerNorm oracle (oracle/layernorm.py).

A slip (variance around 0 instead of the mean, eps outside the root, a
wrong denominator, a dropped correction term in the incremental combine, a
swapped gamma/beta) fails at least one of:
  * torch.nn.functional.layer_norm in float64 on the CPU (the library routine
    the definition reduces to) and a pure-Python math.fsum version;
  * closed forms: a constant row, a two-value row, the affine rescaling rule;
  * invariants: with gamma = 1, beta = 0 the output has mean 0 and mean
    square var / (var + eps); incremental == three-pass for any tiling and tile
    order; a tree of combines equals a flat sequence.
"""
import math

import numpy as np
import pytest
import torch

from oracle.layernorm import combine, layer_norm, layer_norm_incremental, tile_state


def rows(shape, seed, offset=6.0):
    r = np.random.default_rng(seed)
    x = r.standard_normal(shape) * r.uniform(0.5, 2.0, (shape[0], 1)) + r.uniform(-offset, offset, (shape[0], 1))
    g = 1.0 + 0.1 * r.standard_normal(shape[1])
    b = 0.1 * r.standard_normal(shape[1])
    return x, g, b


@pytest.mark.parametrize("H", [1, 2, 7, 64, 1000])
def test_matches_torch_layer_norm(H):
    x, g, b = rows((13, H), H)
    y, mean, rstd = layer_norm(x, g, b, 1e-5)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (H,), torch.tensor(g), torch.tensor(b), 1e-5)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mean, x.mean(axis=1), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(x.var(axis=1) + 1e-5), rtol=1e-12)


def test_matches_pure_python():
    x, g, b = rows((4, 9), 3)
    y, mean, rstd = layer_norm(x, g, b, 1e-3)
    for r in range(4):
        m = math.fsum(x[r]) / 9
        var = math.fsum((v - m) ** 2 for v in x[r]) / 9
        s = 1.0 / math.sqrt(var + 1e-3)
        assert abs(mean[r] - m) <= 1e-14 * max(1.0, abs(m))
        assert abs(rstd[r] - s) <= 1e-13 * s
        for h in range(9):
            assert abs(y[r, h] - ((x[r, h] - m) * s * g[h] + b[h])) <= 1e-12


def test_closed_forms():
    g, b = np.array([2.0, -1.0, 0.5]), np.array([0.25, 0.5, -3.0])
    # constant row: var 0, y = beta
    y, mean, rstd = layer_norm(np.full((1, 3), 7.5), g, b, 1e-4)
    assert mean[0] == 7.5 and rstd[0] == pytest.approx(100.0, rel=1e-14)
    np.testing.assert_array_equal(y[0], b)
    # two values a, b: mean (a+b)/2, var ((a-b)/2)^2, y = -/+ |a-b|/2 * rstd
    y, mean, rstd = layer_norm(np.array([[1.0, 5.0]]), np.ones(2), np.zeros(2), 0.0)
    assert mean[0] == 3.0 and rstd[0] == 0.5
    np.testing.assert_array_equal(y[0], [-1.0, 1.0])


def test_affine_rescaling_rule():
    # LN(s x + t; eps s^2) == LN(x; eps) for s > 0
    x, g, b = rows((5, 33), 4)
    y1, _, _ = layer_norm(x, g, b, 1e-3)
    y2, _, _ = layer_norm(3.0 * x - 11.0, g, b, 1e-3 * 9.0)
    np.testing.assert_allclose(y2, y1, rtol=1e-11, atol=1e-11)


def test_normalised_moments():
    x, _, _ = rows((6, 500), 5)
    eps = 1e-2
    y, _, _ = layer_norm(x, np.ones(500), np.zeros(500), eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((y ** 2).mean(axis=1), var / (var + eps), rtol=1e-12)


@pytest.mark.parametrize("tile", [1, 3, 64, 256, 1000])
def test_incremental_equals_three_pass(tile):
    x, g, b = rows((8, 1000), 6, offset=1e3)   # large offsets: the correction term matters
    y, mean, rstd = layer_norm(x, g, b, 1e-5)
    yi, mi, ri = layer_norm_incremental(x, g, b, 1e-5, tile)
    np.testing.assert_allclose(mi, mean, rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(ri, rstd, rtol=1e-9)
    np.testing.assert_allclose(yi, y, rtol=1e-8, atol=1e-8)


def test_incremental_is_order_independent():
    x, g, b = rows((4, 300), 7)
    y, mean, rstd = layer_norm(x, g, b, 1e-5)
    ntiles = -(-300 // 16)
    for seed in range(3):
        order = np.random.default_rng(seed).permutation(ntiles)
        yi, mi, ri = layer_norm_incremental(x, g, b, 1e-5, 16, order=order)
        np.testing.assert_allclose(yi, y, rtol=1e-10, atol=1e-10)


def test_tree_combine_equals_flat():
    x, _, _ = rows((3, 64), 8)
    parts = [tile_state(x[:, 8 * i:8 * i + 8]) for i in range(8)]
    flat = parts[0]
    for p in parts[1:]:
        flat = combine(flat, p)
    tree = parts
    while len(tree) > 1:
        tree = [combine(tree[i], tree[i + 1]) for i in range(0, len(tree), 2)]
    for a, b in zip(flat, tree[0]):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(flat[2] / 64, x.var(axis=1), rtol=1e-12)
