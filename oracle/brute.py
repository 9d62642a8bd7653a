"""Pure-Python scalar attention for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Written independently of ``cascade.py`` to pin
it: scalar loops, ``math.fsum`` for every sum, the textbook softmax
exp(s_j) / sum_k exp(s_k) without the max shift, and RoPE as multiplication
of the complex number x[i] + 1j*x[i+D/2] by exp(1j * pos * theta_i).
Only valid where exp(s) does not overflow, i.e. for the small scores the
pinning tests use.

Definition followed: the attention pattern of the "Operator Fusion" guide
(section 2, Pattern 4) with the pre-matmul rotation of the AttnFuse listing
(abstract, Fig. 1) and the causal / sliding-window visibility of its Table 6.
"""
from __future__ import annotations

import cmath
import math


def _rot(vec, pos, base):
    D = len(vec)
    half = D // 2
    out = list(vec)
    for i in range(half):
        theta = base ** (-2.0 * i / D)
        z = complex(vec[i], vec[i + half]) * cmath.exp(1j * pos * theta)
        out[i], out[i + half] = z.real, z.imag
    return out


def _visible(p, j, mask, window):
    if mask == "none":
        return True
    if mask == "causal":
        return j <= p
    return p - window < j <= p


def brute_attention(q, k, v, scale, mask="none", window=0, rope_base=0.0, alibi_slopes=None):
    """q: nested lists [B][Hq][Nq][D]; k, v: [B][Hkv][Nk][D].  Returns (O, LSE) lists.

    ALiBi: exp(s) is multiplied by exp(-slope_h * |p - j|), the same as adding
    the bias to the score.
    """
    B, Hq, Nq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Nk = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    O = [[[[0.0] * D for _ in range(Nq)] for _ in range(Hq)] for _ in range(B)]
    L = [[[-math.inf] * Nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Nq):
                p = Nk - Nq + i
                qi = list(q[b][h][i])
                if rope_base > 0:
                    qi = _rot(qi, p, rope_base)
                keys = [j for j in range(Nk) if _visible(p, j, mask, window)]
                if not keys:
                    continue
                ex = []
                for j in keys:
                    kj = list(k[b][g][j])
                    if rope_base > 0:
                        kj = _rot(kj, j, rope_base)
                    s = scale * math.fsum(qi[d] * kj[d] for d in range(D))
                    w = math.exp(s)
                    if alibi_slopes is not None:
                        w *= math.exp(-alibi_slopes[h] * abs(p - j))
                    ex.append(w)
                z = math.fsum(ex)
                for d in range(D):
                    O[b][h][i][d] = math.fsum(ex[n] * v[b][g][j][d] for n, j in enumerate(keys)) / z
                L[b][h][i] = math.log(z)
    return O, L
