"""Plain float64 softmax followed by TopK: a cascade on the max/+ row of
RedFuser's Table 1.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

Sources: RedFuser (Tang et al.), abstract (cascaded reductions, later loops
depending on earlier ones), Table 1 (TopK combines with max and shifts with +,
like Max and ArgMax), Fig. 4 (the incremental form).  The cascade per row x:
  level 1 (max):   m = max_e x_e
  level 2 (+):     l = sum_e exp(x_e - m)                      (reads m)
  level 3 (TopK):  the k largest p_e = exp(x_e - m) / l with their indices
                                                               (reads m and l)

Readings (the pages give no formulas for this cascade):
  * the k largest p_e are the k largest x_e (exp is increasing), so selection
    is done on the exact input values; ties are broken towards the lower index,
    which makes the result unique;
  * values come out in descending order (by the same rule), as float64 here
    and float32 in the kernel; indices as integers;
  * the incremental form keeps (m, l, the k best (x, index) so far): a new
    chunk moves m to m' = max(m, max chunk), l is rescaled by exp(m - m') and
    gets the chunk's sum, and the k best are merged; p is formed at the end.
"""
from __future__ import annotations

import numpy as np

from .cascade import _f64


def _select(x, idx, k):
    """k best of (x, idx) pairs per row: larger x first, then lower index."""
    order = np.lexsort((idx, -x), axis=-1)[..., :k]
    return np.take_along_axis(x, order, -1), np.take_along_axis(idx, order, -1)


def softmax_topk(x, k: int):
    """x [rows, E].  Returns (values [rows, k] float64, indices [rows, k] int64)."""
    x = _f64(x)
    rows, E = x.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    m = x.max(axis=1)                                   # level 1
    l = np.exp(x - m[:, None]).sum(axis=1)              # level 2
    p = np.exp(x - m[:, None]) / l[:, None]             # level 3 input
    idx = np.broadcast_to(np.arange(E), x.shape)
    order = np.lexsort((idx, -x), axis=-1)[:, :k]       # TopK on x (same order as p)
    return np.take_along_axis(p, order, 1), order.astype(np.int64)


def softmax_topk_incremental(x, k: int, chunk: int, order=None):
    """Single pass over column chunks keeping (m, l, k best) per row."""
    x = _f64(x)
    rows, E = x.shape
    starts = list(range(0, E, chunk))
    if order is not None:
        starts = [starts[i] for i in order]
    m = np.full(rows, -np.inf)
    l = np.zeros(rows)
    bx = np.full((rows, 0), -np.inf)
    bi = np.zeros((rows, 0), dtype=np.int64)
    for s in starts:
        c = x[:, s:s + chunk]
        m_new = np.maximum(m, c.max(axis=1))
        alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        l = l * alpha + np.exp(c - m_new[:, None]).sum(axis=1)
        m = m_new
        cand_x = np.concatenate([bx, c], axis=1)
        cand_i = np.concatenate([bi, np.broadcast_to(np.arange(s, s + c.shape[1]), c.shape)], axis=1)
        bx, bi = _select(cand_x, cand_i, min(k, cand_x.shape[1]))
    return np.exp(bx - m[:, None]) / l[:, None], bi
