"""Plain float64 LayerNorm: a second cascaded reduction (mean, then variance).

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

Sources:
  * "Operator Fusion" guide, section 2, Pattern 2 (reduction + element-wise):
    LayerNorm as pass 1 mean, pass 2 variance around that mean, pass 3 the
    element-wise normalisation (x - mean) / sqrt(var) * gamma + beta.
  * RedFuser (Tang et al.), abstract and Table 1: a cascade of reductions
    whose later level depends on an earlier level's result, here + for the
    mean and + for the squared deviations, which depend on the mean; Fig. 4:
    the incremental form that updates every level as each input tile arrives.

Readings (the pages give no formulas for these):
  * eps is added to the variance inside the square root, as in the usual
    LayerNorm; var is the population variance (divide by H);
  * the incremental form keeps (n, mean, M2) per row, M2 = sum of squared
    deviations from the running mean.  A new tile (n_b, mean_b, M2_b) moves the
    level-1 result by delta = mean_b - mean_a, and the level-2 result gets the
    correction delta^2 n_a n_b / n (the role exp(m_old - m_new) plays for the
    softmax cascade): the pairwise update of Chan, Golub and LeVeque.
"""
from __future__ import annotations

import numpy as np

from .cascade import _f64


def layer_norm(x, gamma, beta, eps: float):
    """x [rows, H]; gamma, beta [H].  Returns (y [rows, H], mean [rows], rstd [rows]).

    Pass 1 (combine +):  mean = sum_h x / H
    Pass 2 (combine +):  var  = sum_h (x - mean)^2 / H       (reads pass 1)
    Pass 3 (element-wise): y = (x - mean) * rstd * gamma + beta,  rstd = 1/sqrt(var + eps)
    """
    x, gamma, beta = _f64(x), _f64(gamma), _f64(beta)
    H = x.shape[-1]
    mean = x.sum(axis=-1) / H
    var = ((x - mean[..., None]) ** 2).sum(axis=-1) / H
    rstd = 1.0 / np.sqrt(var + eps)
    y = (x - mean[..., None]) * rstd[..., None] * gamma + beta
    return y, mean, rstd


def combine(a, b):
    """Merge two partial states (n, mean, M2) of the same row (arrays allowed)."""
    na, ma, Ma = a
    nb, mb, Mb = b
    n = na + nb
    with np.errstate(invalid="ignore", divide="ignore"):
        delta = mb - ma
        wb = np.where(n > 0, nb / np.where(n > 0, n, 1), 0.0)
        mean = ma + delta * wb
        M2 = Ma + Mb + delta * delta * np.where(n > 0, na * nb / np.where(n > 0, n, 1), 0.0)
    return n, mean, M2


def tile_state(t):
    """(n, mean, M2) of one tile t [rows, w] by its own two passes."""
    n = np.full(t.shape[0], float(t.shape[-1]))
    mean = t.sum(axis=-1) / t.shape[-1]
    return n, mean, ((t - mean[:, None]) ** 2).sum(axis=-1)


def layer_norm_incremental(x, gamma, beta, eps: float, tile: int, order=None):
    """Single pass over column tiles of width ``tile`` keeping only (n, mean, M2)
    per row; ``order`` permutes the tiles (the result must not depend on it)."""
    x, gamma, beta = _f64(x), _f64(gamma), _f64(beta)
    rows, H = x.shape
    starts = list(range(0, H, tile))
    if order is not None:
        starts = [starts[i] for i in order]
    state = (np.zeros(rows), np.zeros(rows), np.zeros(rows))
    for s in starts:
        state = combine(state, tile_state(x[:, s:s + tile]))
    n, mean, M2 = state
    rstd = 1.0 / np.sqrt(M2 / n + eps)
    y = (x - mean[:, None]) * rstd[:, None] * gamma + beta
    return y, mean, rstd
