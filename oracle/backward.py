"""Plain float64 gradients of the attention forward defined in ``cascade.py``.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

What the pages fix: AttnFuse (abstract; Table 9) runs the same attention
variants inside a training step, forward then backward then optimiser step,
so the backward of the fused forward is the next step on the path.  The pages
print no backward formulas; what follows is the chain rule applied to the
forward definition (cascade.py), and nothing else:

    q' = R(p_i) q_i,  k' = R(j) k_j           (RoPE, when on; R is a rotation)
    s_ij = scale * q'_i . k'_j + b_ij          (b = ALiBi bias, input-independent)
    P_ij = exp(s_ij) / sum_visible exp(s_ik)   (0 where j is not visible)
    O_i  = sum_j P_ij v_j

Given dO (the gradient of a scalar loss with respect to O; LSE is taken as
not feeding the loss):

    dV_j   = sum_i P_ij dO_i                   (summed over the query heads
                                                that share the KV head)
    dP_ij  = dO_i . v_j
    D_i    = sum_j P_ij dP_ij                  (softmax Jacobian: row term)
    dS_ij  = P_ij (dP_ij - D_i)
    dq'_i  = scale * sum_j dS_ij k'_j,   dq_i = R(p_i)^T dq'_i
    dk'_j  = scale * sum_i dS_ij q'_i,   dk_j = R(j)^T dk'_j

R(pos)^T is the rotation by -pos * theta_i.  Rows with no visible key have
P = 0 and contribute nothing.  The slopes of ALiBi get no gradient.
"""
from __future__ import annotations

import numpy as np

from .cascade import (NEG_INF, _f64, alibi_bias, query_positions, rope_rotate, visible_mask)


def _probs(s):
    """Three passes over masked scores s [R, K]: max, exp-sum, normalise."""
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], NEG_INF)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    return e / np.where(l > 0, l, 1.0)[:, None]


def attention_backward(q, k, v, do, scale, mask="none", window=0, rope_base=0.0, alibi_slopes=None,
                       heads=None):
    """Returns (dq [B,Hq,Nq,D], dk [B,Hkv,Nk,D], dv [B,Hkv,Nk,D]) in float64.

    ``heads``: optional iterable of (b, h) query heads to include; the others
    contribute nothing (their dq stays 0 and their share of dk, dv is left
    out).  Used to check one KV group at full size.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    pq, pk = query_positions(Nq, Nk), np.arange(Nk)
    vis = visible_mask(pq, pk, mask, window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    for b, h in todo:
        g = h // G
        qr, kr = q[b, h], k[b, g]
        if rope_base > 0:
            qr, kr = rope_rotate(qr, pq, rope_base), rope_rotate(kr, pk, rope_base)
        s = scale * (qr @ kr.T)
        if alibi_slopes is not None:
            s = s + alibi_bias(alibi_slopes[h], pq, pk)
        P = _probs(np.where(vis, s, NEG_INF))
        dv[b, g] += P.T @ do[b, h]
        dP = do[b, h] @ v[b, g].T
        Drow = (P * dP).sum(axis=1)
        dS = P * (dP - Drow[:, None])
        dqr = scale * (dS @ kr)
        dkr = scale * (dS.T @ qr)
        if rope_base > 0:
            dqr = rope_rotate(dqr, -pq, rope_base)   # R(p)^T = R(-p)
            dkr = rope_rotate(dkr, -pk, rope_base)
        dq[b, h] = dqr
        dk[b, g] += dkr
    return dq, dk, dv


def row_terms(o, do):
    """D_i = dO_i . O_i for every row: equals sum_j P_ij dP_ij when O is the
    exact forward output (O_i = sum_j P_ij v_j), which is how a kernel can get
    the softmax row term from the saved output instead of recomputing P."""
    return (_f64(o) * _f64(do)).sum(axis=-1)
