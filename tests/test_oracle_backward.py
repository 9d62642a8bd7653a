"""Pins for the float64 attention backward (oracle/backward.py).

A slip in the gradient formulas (a dropped softmax row term, a missing
scale, a transposed dS, the forward rather than the inverse rotation, GQA
gradients not summed over the group) fails at least one of:
  * central finite differences of the pure-Python brute-force forward
    (oracle/brute.py, written independently of the vectorised oracle);
  * torch autograd in float64 through a forward written here with torch ops;
  * invariants: sum_j dv_j = sum of dO over rows that see a key; sum_j dk_j = 0
    without RoPE (rows of dS sum to zero); a row that sees one key has dq = 0;
    scale 0 gives dq = dk = 0 and dv = P^T dO with uniform P.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import cascade as A
from oracle.backward import attention_backward, row_terms
from oracle.brute import brute_attention


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def loss_brute(q, k, v, do, scale, mask, window, base, slopes):
    o, _ = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, mask, window, base, slopes)
    return float(np.sum(np.array(o) * do))


FD_CASES = [
    # (B, Hq, Hkv, Nq, Nk, D, mask, window, rope_base, alibi)
    (1, 1, 1, 4, 4, 4, "none", 0, 0.0, False),
    (1, 2, 1, 4, 5, 4, "causal", 0, 0.0, False),      # GQA 2:1, Nq < Nk
    (1, 1, 1, 5, 5, 2, "sliding", 2, 0.0, False),
    (1, 2, 2, 4, 4, 4, "causal", 0, 100.0, False),    # RoPE
    (1, 2, 1, 3, 5, 4, "sliding", 3, 50.0, False),    # RoPE + window + GQA
    (1, 2, 2, 4, 4, 2, "causal", 0, 0.0, True),       # ALiBi
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,D,mask,window,base,alibi", FD_CASES)
def test_gradients_match_finite_differences_of_brute_force(B, Hq, Hkv, Nq, Nk, D, mask, window, base, alibi):
    seed = zlib.crc32(repr((B, Hq, Hkv, Nq, Nk, D, mask, window, base, alibi)).encode())
    q, k, v = rnd((B, Hq, Nq, D), seed), rnd((B, Hkv, Nk, D), seed + 1), rnd((B, Hkv, Nk, D), seed + 2)
    do = rnd((B, Hq, Nq, D), seed + 3)
    scale = 0.7
    slopes = [0.5 * (h + 1) for h in range(Hq)] if alibi else None
    dq, dk, dv = attention_backward(q, k, v, do, scale, mask, window, base, slopes)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = x[idx]
            x[idx] = x0 + eps
            lp = loss_brute(q, k, v, do, scale, mask, window, base, slopes)
            x[idx] = x0 - eps
            lm = loss_brute(q, k, v, do, scale, mask, window, base, slopes)
            x[idx] = x0
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (idx, fd, g[idx])


def torch_forward(q, k, v, scale, mask, window, base, slopes):
    """Forward with plain torch ops (float64), for autograd."""
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    pq = torch.arange(Nq, dtype=torch.float64) + (Nk - Nq)
    pk = torch.arange(Nk, dtype=torch.float64)

    def rot(x, pos):
        half = D // 2
        theta = base ** (-2.0 * torch.arange(half, dtype=torch.float64) / D)
        a = pos[:, None] * theta[None, :]
        x1, x2 = x[..., :half], x[..., half:]
        return torch.cat([x1 * torch.cos(a) - x2 * torch.sin(a), x1 * torch.sin(a) + x2 * torch.cos(a)], dim=-1)

    if base > 0:
        q, k = rot(q, pq), rot(k, pk)
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    s = scale * torch.matmul(q, k.transpose(-1, -2))
    if slopes is not None:
        s = s - torch.tensor(slopes, dtype=torch.float64)[None, :, None, None] * (pq[:, None] - pk[None, :]).abs()
    vis = torch.ones(Nq, Nk, dtype=torch.bool)
    if mask != "none":
        vis = pk[None, :] <= pq[:, None]
        if mask == "sliding":
            vis &= pk[None, :] > pq[:, None] - window
    s = s.masked_fill(~vis, -math.inf)
    p = torch.softmax(s, dim=-1).nan_to_num(0.0)  # rows with no key: 0
    return torch.matmul(p, v)


AG_CASES = [
    (2, 4, 2, 33, 47, 8, "causal", 0, 0.0, False),
    (1, 2, 2, 40, 40, 16, "none", 0, 10000.0, False),
    (1, 4, 1, 30, 50, 8, "sliding", 9, 10000.0, False),
    (1, 2, 2, 25, 25, 8, "causal", 0, 0.0, True),
    (1, 2, 1, 12, 6, 4, "causal", 0, 0.0, False),       # Nq > Nk: early rows see nothing
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,D,mask,window,base,alibi", AG_CASES)
def test_gradients_match_torch_autograd(B, Hq, Hkv, Nq, Nk, D, mask, window, base, alibi):
    seed = zlib.crc32(repr((B, Hq, Hkv, Nq, Nk, D, mask, window, base, alibi)).encode())
    q, k, v = rnd((B, Hq, Nq, D), seed), rnd((B, Hkv, Nk, D), seed + 1), rnd((B, Hkv, Nk, D), seed + 2)
    do = rnd((B, Hq, Nq, D), seed + 3)
    scale = 1.0 / math.sqrt(D)
    slopes = [2.0 ** (-(h + 1)) for h in range(Hq)] if alibi else None
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch_forward(tq, tk, tv, scale, mask, window, base, slopes)
    o.backward(torch.tensor(do))
    dq, dk, dv = attention_backward(q, k, v, do, scale, mask, window, base, slopes)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 6)])
def test_gradient_invariants(mask, window):
    B, Hq, Hkv, Nq, Nk, D = 2, 4, 2, 20, 26, 8
    q, k, v, do = rnd((B, Hq, Nq, D), 1), rnd((B, Hkv, Nk, D), 2), rnd((B, Hkv, Nk, D), 3), rnd((B, Hq, Nq, D), 4)
    dq, dk, dv = attention_backward(q, k, v, do, 0.4, mask, window)
    pq = A.query_positions(Nq, Nk)
    seen = A.visible_mask(pq, np.arange(Nk), mask, window).any(axis=1)  # rows with a key
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            # columns of P sum (over rows that see a key) to ... rows of P sum to 1
            want = sum(do[b, h][seen].sum(axis=0) for h in range(g * G, (g + 1) * G))
            np.testing.assert_allclose(dv[b, g].sum(axis=0), want, rtol=1e-12, atol=1e-12)
            # rows of dS sum to zero, so the key gradients cancel (no RoPE)
            np.testing.assert_allclose(dk[b, g].sum(axis=0), 0.0, atol=1e-12)
    # a row that sees exactly one key has P = 1 there and dS = 0
    one = A.visible_mask(pq, np.arange(Nk), mask, window).sum(axis=1) == 1
    if one.any():
        assert np.all(dq[:, :, one] == 0.0)


def test_scale_zero_gives_uniform_weights_and_no_score_gradient():
    q, k, v, do = rnd((1, 2, 9, 4), 5), rnd((1, 2, 9, 4), 6), rnd((1, 2, 9, 4), 7), rnd((1, 2, 9, 4), 8)
    dq, dk, dv = attention_backward(q, k, v, do, 0.0, "causal")
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    # P_ij = 1/(i+1) for j <= i
    P = np.tril(np.ones((9, 9))) / np.arange(1, 10)[:, None]
    for h in range(2):
        np.testing.assert_allclose(dv[0, h], P.T @ do[0, h], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("base", [0.0, 10000.0])
def test_row_term_from_saved_output(base):
    q, k, v, do = rnd((1, 2, 15, 8), 9), rnd((1, 1, 15, 8), 10), rnd((1, 1, 15, 8), 11), rnd((1, 2, 15, 8), 12)
    o, _ = oracle.attention(q, k, v, 0.3, "causal", rope_base=base)
    for h in range(2):
        P = oracle.softmax_probs(q, k, 0.3, "causal", rope_base=base, b=0, h=h)
        dP = do[0, h] @ v[0, 0].T
        np.testing.assert_allclose(row_terms(o, do)[0, h], (P * dP).sum(axis=1), rtol=1e-12, atol=1e-12)


def test_heads_subset_matches_full():
    q, k, v, do = rnd((1, 4, 10, 4), 13), rnd((1, 2, 12, 4), 14), rnd((1, 2, 12, 4), 15), rnd((1, 4, 10, 4), 16)
    full = attention_backward(q, k, v, do, 0.5, "causal", rope_base=100.0)
    part = attention_backward(q, k, v, do, 0.5, "causal", rope_base=100.0, heads=[(0, 2), (0, 3)])
    np.testing.assert_array_equal(part[0][:, 2:], full[0][:, 2:])
    np.testing.assert_allclose(part[1][:, 1], full[1][:, 1], rtol=0, atol=0)
    np.testing.assert_allclose(part[2][:, 1], full[2][:, 1], rtol=0, atol=0)
