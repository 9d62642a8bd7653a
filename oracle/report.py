"""Whole-output comparison of a kernel's attention result with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).  The oracle is
evaluated one (batch, KV head) group at a time, over every query head of that
group and every query row, so a full-size workload never needs its whole
float64 copy in memory at once.  Each group's exact O and LSE are compared
element by element with the kernel's, and the per-group figures of
``cascade.error_report`` are folded into one report: the largest |O - O64|
and |LSE - LSE64|, the rounding floor max |rn(O64) - O64| (what rounding the
exact output once to the output dtype costs), the largest distance from
rn(O64) in units of the output grid's spacing, and where the largest O error
sits.
"""
from __future__ import annotations

import time

import numpy as np

from . import cascade as A


def _merge(total, part, b, h0):
    if total is None:
        total = dict(part)
        total["worst"] = dict(part["worst"])
        total["worst"]["index"] = [b, h0 + part["worst"]["index"][0]] + part["worst"]["index"][1:]
        return total
    if part["max_abs_o"] > total["max_abs_o"]:
        total["worst"] = dict(part["worst"])
        total["worst"]["index"] = [b, h0 + part["worst"]["index"][0]] + part["worst"]["index"][1:]
    for key in ("max_abs_o", "max_abs_lse", "floor", "ulps"):
        total[key] = max(total[key], part[key])
    return total


def attention_by_group(q, k, v, scale, mask="none", window=0, rope_base=0.0, row_block=None):
    """Yield (b, g, O64 [G, Nq, D], LSE64 [G, Nq]) for every batch b and KV head g:
    the oracle's three-pass cascade for the G = Hq/Hkv query heads that read
    KV head g.  q, k, v may live on any device; each group's slices are copied
    to the CPU (exactly) before use."""
    B, Hq, Nq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if row_block is None:
        # the sliding window's key span per block is rows + window - 1
        row_block = 128 if mask == "sliding" and window <= 1024 else 512
    for b in range(B):
        for g in range(Hkv):
            o, lse = A.attention(q[b:b + 1, g * G:(g + 1) * G], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                                 scale, mask, window, rope_base, row_block=row_block)
            yield b, g, o[0], lse[0]


def compare_full(q, k, v, o, lse, scale, mask, window, rope_base, out_dtype):
    """Report (dict) of the kernel's (o [B,Hq,Nq,D], lse [B,Hq,Nq]) against the
    oracle over every element, plus the oracle's own wall time in seconds
    ("oracle_s", slice copies excluded).  ``out_dtype`` is o's torch dtype."""
    G = q.shape[1] // k.shape[1]
    total, t_oracle = None, 0.0
    groups = attention_by_group(q, k, v, scale, mask, window, rope_base)
    while True:
        t0 = time.perf_counter()
        try:
            b, g, o64, l64 = next(groups)
        except StopIteration:
            break
        t_oracle += time.perf_counter() - t0
        h0 = g * G
        part = A.error_report(o[b, h0:h0 + G], lse[b, h0:h0 + G], o64, l64, out_dtype)
        # every row the oracle gives -inf must be -inf in the kernel's lse too
        kl = A._f64(lse[b, h0:h0 + G])
        fin = np.isfinite(l64)
        if not np.array_equal(np.isfinite(kl), fin) or not np.all(kl[~fin] == -np.inf):
            part["max_abs_lse"] = float("inf")
        if not np.all(np.isfinite(A._f64(o[b, h0:h0 + G]))):
            part["max_abs_o"] = float("inf")
        total = _merge(total, part, b, h0)
    total["oracle_s"] = t_oracle
    return total


def compare_partials(q, k, v, o_part, lse_part, scale, num_splits, mask="none", window=0, rope_base=0.0):
    """Largest |o_c - O_c| and |lse_c - LSE_c| over every split-KV partial
    (chunks with no visible key must hold o_c = 0 and lse_c = -inf)."""
    B, Hq = q.shape[:2]
    Hkv = k.shape[1]
    G = Hq // Hkv
    err_o = err_l = 0.0
    for b in range(B):
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            op, lp = A.split_partials(q[b:b + 1, hs], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                                      scale, num_splits, mask, window, rope_base)
            ko, kl = A._f64(o_part[b:b + 1, hs]), A._f64(lse_part[b:b + 1, hs])
            fin = np.isfinite(lp)
            if not np.array_equal(np.isfinite(kl), fin) or not np.all(kl[~fin] == -np.inf):
                return float("inf"), float("inf")
            err_o = max(err_o, float(np.abs(ko - op).max()))
            if fin.any():
                err_l = max(err_l, float(np.abs(kl[fin] - lp[fin]).max()))
    return err_o, err_l
