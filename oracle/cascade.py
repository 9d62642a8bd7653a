"""Plain, slow, float64 definition of what the fused attention kernels compute.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path may import this module.

Sources (cited by page title and the part of the page):
  * "RedFuser: An Automatic Operator Fusion Framework for Cascaded Reductions
    on AI Accelerators" (Tang et al.): abstract (safe softmax followed by a
    GEMM is a cascaded reduction), Fig. 3 (fused and unfused forms compute the
    same result), Fig. 4 (incremental form: each level is updated as input
    arrives), Table 1 (max/+ and +/* operator pairs), Fig. 13 (FlashDecoding).
  * "AttnFuse: A Composable DSL for Compiling Attentions to Fused GPU Kernels"
    (Dasoju, Zhao): abstract and Fig. 1 (RoPE is applied to Q and K before the
    central matmul), Table 6 (causal, sliding window W=256), Table 8 (decode
    with 32 query heads over 8 KV heads).
  * "Operator Fusion" guide, section 2, Pattern 4 (scores = Q K^T / sqrt(dk),
    mask, softmax, times V).

Readings where the pages are silent:
  * query row i sits at position p_i = Nk - Nq + i; key row j at position j
    (bottom-right alignment; equals i when Nq == Nk);
  * causal: key j visible iff j <= p_i; sliding window W: p_i - W < j <= p_i;
  * a row with no visible key has O = 0 and LSE = -inf;
  * LSE is the natural log of sum_j exp(s_ij) over visible j, scores scaled;
  * RoPE: half-split pairs (x[i], x[i + D/2]), theta_i = base^(-2i/D), angle
    = position * theta_i, rotation by +angle; applied to q and k only, before
    the scale; V is not rotated;
  * GQA: query head h reads KV head h // (Hq // Hkv);
  * split-KV chunk c covers keys [c*ceil(Nk/S), min(Nk, (c+1)*ceil(Nk/S)));
  * ALiBi (AttnFuse Table 6 names "Causal+ALiBi" only): a per-head slope m_h
    adds the bias -m_h * |p_i - j| to the scaled score of every visible pair;
    the slopes are an input.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor or array-like to a float64 numpy array."""
    if hasattr(x, "detach"):
        import torch  # local: only to read tensors handed in by the caller
        x = x.detach().to("cpu")
        if x.dtype in (torch.float16, torch.bfloat16):
            x = x.to(torch.float32)  # exact: both embed in float32
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# RoPE, pre-matmul (AttnFuse abstract and Fig. 1)
# --------------------------------------------------------------------------
def rope_rotate(x, positions, base: float) -> np.ndarray:
    """Rotate half-split pairs of the last axis by position * theta_i.

    x: [..., N, D] (D even), positions: [N].  For i in [0, D/2):
        theta_i = base ** (-2 i / D),  a = pos * theta_i
        x'[i]       = x[i] cos a - x[i + D/2] sin a
        x'[i + D/2] = x[i] sin a + x[i + D/2] cos a
    """
    x = _f64(x)
    D = x.shape[-1]
    if D % 2:
        raise ValueError("RoPE needs an even head dimension")
    half = D // 2
    i = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * i / D)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]  # [N, D/2]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, lo * s + hi * c], axis=-1)


# --------------------------------------------------------------------------
# Visibility (AttnFuse Table 6: causal and sliding window)
# --------------------------------------------------------------------------
def query_positions(Nq: int, Nk: int) -> np.ndarray:
    return np.arange(Nq, dtype=np.int64) + (Nk - Nq)


def visible_mask(pos_q, pos_k, mask: str, window: int = 0) -> np.ndarray:
    """Boolean [len(pos_q), len(pos_k)]: True where key j is visible to query i."""
    pq = np.asarray(pos_q, dtype=np.int64)[:, None]
    pk = np.asarray(pos_k, dtype=np.int64)[None, :]
    if mask == "none":
        return np.ones((pq.shape[0], pk.shape[1]), dtype=bool)
    if mask == "causal":
        return pk <= pq
    if mask == "sliding":
        if window < 1:
            raise ValueError("sliding window needs window >= 1")
        return (pk <= pq) & (pk > pq - window)
    raise ValueError(f"unknown mask {mask!r}")


def _key_span(p_lo: int, p_hi: int, Nk: int, mask: str, window: int):
    """Smallest key range [lo, hi) holding every key visible to positions p_lo..p_hi."""
    if mask == "none":
        return 0, Nk
    hi = min(Nk, p_hi + 1)
    lo = 0 if mask == "causal" else max(0, p_lo - window + 1)
    return lo, max(lo, hi)


def alibi_bias(slope: float, pos_q, pos_k) -> np.ndarray:
    """ALiBi bias -slope * |p_i - j| for query positions pos_q and key positions pos_k."""
    pq = np.asarray(pos_q, dtype=np.float64)[:, None]
    pk = np.asarray(pos_k, dtype=np.float64)[None, :]
    return -float(slope) * np.abs(pq - pk)


# --------------------------------------------------------------------------
# The unfused three-pass cascade (RedFuser abstract, Fig. 3a; guide Pattern 4)
# --------------------------------------------------------------------------
def _three_pass(qr, kr, v, vis, scale, bias=None):
    """One head, a block of query rows.  qr [R, D], kr [K, D], v [K, D], vis [R, K],
    bias [R, K] (ALiBi) or None.

    Level 1 (combine = max):        m_i = max_j s_ij
    Level 2 (combine = +):          l_i = sum_j exp(s_ij - m_i)
    Level 3 (combine = +, op = *):  O_i = sum_j (exp(s_ij - m_i) / l_i) v_j
    Each level is a full pass over the scores that reads the previous level's result.
    """
    s = scale * (qr @ kr.T)
    if bias is not None:
        s = s + bias
    s = np.where(vis, s, NEG_INF)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], NEG_INF)   # pass 1
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])                                       # masked -> 0
    l = e.sum(axis=1)                                                     # pass 2
    l_safe = np.where(empty, 1.0, l)
    o = (e / l_safe[:, None]) @ v                                         # pass 3
    o[empty] = 0.0
    lse = np.where(empty, NEG_INF, m_safe + np.log(l_safe))
    return o, lse


def softmax_probs(q, k, scale, mask="none", window=0, rope_base=0.0, b=0, h=0, alibi_slopes=None):
    """Dense P = softmax(masked scaled scores) for one head, via the first two passes.

    Returned for the invariant that every row with a visible key sums to one.
    """
    q, k = _f64(q), _f64(k)
    Hq, Nq, Nk = q.shape[1], q.shape[2], k.shape[2]
    g = h // (Hq // k.shape[1])
    pq, pk = query_positions(Nq, Nk), np.arange(Nk)
    qr, kr = q[b, h], k[b, g]
    if rope_base > 0:
        qr, kr = rope_rotate(qr, pq, rope_base), rope_rotate(kr, pk, rope_base)
    sc = scale * (qr @ kr.T)
    if alibi_slopes is not None:
        sc = sc + alibi_bias(alibi_slopes[h], pq, pk)
    s = np.where(visible_mask(pq, pk, mask, window), sc, NEG_INF)
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    return e / np.where(l > 0, l, 1.0)[:, None]


def attention(q, k, v, scale, mask="none", window=0, rope_base=0.0,
              key_lo=0, key_hi=None, row_block=512, alibi_slopes=None):
    """Full forward: returns (O [B,Hq,Nq,D], LSE [B,Hq,Nq]) in float64.

    Works one (b, h) at a time, in blocks of query rows, over exactly the key
    range those rows can see (masked terms are exactly zero, so this is the
    same sum).  ``key_lo``/``key_hi`` further restrict the keys to one split-KV
    chunk; keys outside are treated as not visible.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    key_hi = Nk if key_hi is None else min(key_hi, Nk)
    pq = query_positions(Nq, Nk)
    O = np.zeros((B, Hq, Nq, D))
    L = np.full((B, Hq, Nq), NEG_INF)
    kr_cache = {}
    for b in range(B):
        for h in range(Hq):
            g = h // G
            if (b, g) not in kr_cache:
                kr_cache.clear()
                kr = k[b, g]
                if rope_base > 0:
                    kr = rope_rotate(kr, np.arange(Nk), rope_base)
                kr_cache[(b, g)] = kr
            kr = kr_cache[(b, g)]
            qh = q[b, h]
            if rope_base > 0:
                qh = rope_rotate(qh, pq, rope_base)
            for r0 in range(0, Nq, row_block):
                r1 = min(Nq, r0 + row_block)
                lo, hi = _key_span(int(pq[r0]), int(pq[r1 - 1]), Nk, mask, window)
                lo, hi = max(lo, key_lo), min(hi, key_hi)
                if hi <= lo:
                    continue  # no visible key: O = 0, LSE = -inf already
                vis = visible_mask(pq[r0:r1], np.arange(lo, hi), mask, window)
                bias = None if alibi_slopes is None else alibi_bias(alibi_slopes[h], pq[r0:r1], np.arange(lo, hi))
                o, lse = _three_pass(qh[r0:r1], kr[lo:hi], v[b, g, lo:hi], vis, scale, bias)
                O[b, h, r0:r1], L[b, h, r0:r1] = o, lse
    return O, L


def attention_rows(q, k, v, scale, rows, mask="none", window=0, rope_base=0.0, alibi_slopes=None):
    """O and LSE for selected rows only: ``rows`` is an iterable of (b, h, i).

    Returns (O [R, D], LSE [R]) in the order given.  Each row is the same
    three-pass definition over that one query row's visible keys.
    """
    qf, kf, vf = q, k, v
    Hq, Nq = qf.shape[1], qf.shape[2]
    Hkv, Nk = kf.shape[1], kf.shape[2]
    G = Hq // Hkv
    pq = query_positions(Nq, Nk)
    rows = [tuple(int(t) for t in r) for r in rows]
    out_o = np.zeros((len(rows), qf.shape[3]))
    out_l = np.full(len(rows), NEG_INF)
    for n, (b, h, i) in enumerate(rows):
        g = h // G
        p = int(pq[i])
        lo, hi = _key_span(p, p, Nk, mask, window)
        if hi <= lo:
            continue
        qi = _f64(qf[b, h, i:i + 1])
        kr = _f64(kf[b, g, lo:hi])
        if rope_base > 0:
            qi = rope_rotate(qi, np.array([p]), rope_base)
            kr = rope_rotate(kr, np.arange(lo, hi), rope_base)
        vis = visible_mask(np.array([p]), np.arange(lo, hi), mask, window)
        bias = None if alibi_slopes is None else alibi_bias(alibi_slopes[h], [p], np.arange(lo, hi))
        o, lse = _three_pass(qi, kr, _f64(vf[b, g, lo:hi]), vis, scale, bias)
        out_o[n], out_l[n] = o[0], lse[0]
    return out_o, out_l


# --------------------------------------------------------------------------
# Incremental form (RedFuser Fig. 4b; operator pairs of Table 1)
# --------------------------------------------------------------------------
def attention_incremental(q, k, v, scale, mask="none", window=0, rope_base=0.0,
                          tile=64, order=None, alibi_slopes=None):
    """Single pass over key tiles, keeping only the running (m, l, O) per row.

    For each tile T of keys, with s the tile's masked scaled scores:
        m' = max(m, max_{j in T} s_j)
        a  = exp(m - m')              (a = 0 when m = -inf)
        l  = a l + sum_{j in T} exp(s_j - m')
        O  = a O + sum_{j in T} exp(s_j - m') v_j
    and finally O / l, LSE = m + ln l.  A row whose m' is still -inf keeps its
    state (nothing visible yet).  ``order`` optionally permutes the tiles.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    pq, pk = query_positions(Nq, Nk), np.arange(Nk)
    tiles = [np.arange(t0, min(Nk, t0 + tile)) for t0 in range(0, Nk, tile)]
    if order is not None:
        tiles = [tiles[t] for t in order]
    O = np.zeros((B, Hq, Nq, D))
    L = np.full((B, Hq, Nq), NEG_INF)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            qh, kh = q[b, h], k[b, g]
            if rope_base > 0:
                qh, kh = rope_rotate(qh, pq, rope_base), rope_rotate(kh, pk, rope_base)
            m = np.full(Nq, NEG_INF)
            l = np.zeros(Nq)
            acc = np.zeros((Nq, D))
            for T in tiles:
                vis = visible_mask(pq, T, mask, window)
                sc = scale * (qh @ kh[T].T)
                if alibi_slopes is not None:
                    sc = sc + alibi_bias(alibi_slopes[h], pq, T)
                s = np.where(vis, sc, NEG_INF)
                m_new = np.maximum(m, s.max(axis=1))
                live = np.isfinite(m_new)
                m_ref = np.where(live, m_new, 0.0)
                a = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
                a = np.where(live, a, 1.0)
                p = np.exp(s - m_ref[:, None])
                l = a * l + p.sum(axis=1)
                acc = a[:, None] * acc + p @ v[b, g][T]
                m = m_new
            ok = l > 0
            O[b, h] = np.where(ok[:, None], acc / np.where(ok, l, 1.0)[:, None], 0.0)
            L[b, h] = np.where(ok, m + np.log(np.where(ok, l, 1.0)), NEG_INF)
    return O, L


# --------------------------------------------------------------------------
# Split-KV partials and their log-sum-exp merge (RedFuser Fig. 13)
# --------------------------------------------------------------------------
def split_bounds(Nk: int, num_splits: int):
    step = -(-Nk // num_splits)
    return [(c * step, min(Nk, (c + 1) * step)) for c in range(num_splits)]


def split_partials(q, k, v, scale, num_splits, mask="none", window=0, rope_base=0.0, alibi_slopes=None):
    """Per-chunk normalised partials: (O_c [B,Hq,Nq,S,D], lse_c [B,Hq,Nq,S]).

    Chunk c is the three-pass definition restricted to its key range; a chunk
    with no visible key gives O_c = 0 and lse_c = -inf.
    """
    q = _f64(q)
    B, Hq, Nq, D = q.shape
    Nk = k.shape[2]
    Op = np.zeros((B, Hq, Nq, num_splits, D))
    Lp = np.full((B, Hq, Nq, num_splits), NEG_INF)
    for c, (lo, hi) in enumerate(split_bounds(Nk, num_splits)):
        if hi <= lo:
            continue
        o, lse = attention(q, k, v, scale, mask, window, rope_base, key_lo=lo, key_hi=hi,
                           alibi_slopes=alibi_slopes)
        Op[:, :, :, c], Lp[:, :, :, c] = o, lse
    return Op, Lp


def lse_merge(o_parts, lse_parts):
    """Merge normalised partials along the second-to-last / last axis.

    o_parts [..., S, D], lse_parts [..., S]:
        M   = max_c lse_c
        lse = M + ln sum_c exp(lse_c - M)
        O   = sum_c exp(lse_c - lse) O_c
    All chunks empty: O = 0, lse = -inf.
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    M = lse_parts.max(axis=-1)
    live = np.isfinite(M)
    M_safe = np.where(live, M, 0.0)
    w = np.exp(lse_parts - M_safe[..., None])          # -inf chunks -> 0
    tot = w.sum(axis=-1)
    lse = np.where(live, M_safe + np.log(np.where(live, tot, 1.0)), NEG_INF)
    lse_safe = np.where(live, lse, 0.0)
    wn = np.where(live[..., None], np.exp(lse_parts - lse_safe[..., None]), 0.0)
    O = (wn[..., None] * o_parts).sum(axis=-2)
    return O, lse


# --------------------------------------------------------------------------
# Output rounding: what a kernel that rounds the exact result once would err
# --------------------------------------------------------------------------
def round_to(o64, dtype) -> np.ndarray:
    """rn_dtype(O): the float64 values rounded once, to nearest even, to ``dtype``
    (a torch dtype), returned as float64."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(_f64(o64)))
    return t.to(dtype).to(torch.float64).numpy()


def rounding_floor(o64: np.ndarray, dtype) -> float:
    """max |rn_dtype(O) - O|: the error that rounding the exact output alone makes."""
    o64 = _f64(o64)
    return float(np.abs(round_to(o64, dtype) - o64).max()) if o64.size else 0.0


# significand bits (hidden bit included) and exponent of the smallest normal
_FORMAT = {"float16": (11, -14), "bfloat16": (8, -126), "float32": (24, -126)}


def output_ulp(x, dtype) -> np.ndarray:
    """Spacing of ``dtype``'s grid at each value of x (values of that grid, as
    float64): 2^(e - p + 1) for |x| in [2^e, 2^(e+1)) with p significand bits,
    and the subnormal spacing below the smallest normal."""
    name = str(dtype).replace("torch.", "")
    p, emin = _FORMAT[name]
    a = np.abs(_f64(x))
    _, e = np.frexp(np.where(a > 0, a, 1.0))   # a = m 2^e, m in [0.5, 1)
    e = np.maximum(e - 1, emin)
    return np.ldexp(1.0, e - p + 1)


def error_report(o, lse, o64, lse64, dtype) -> dict:
    """Error of a kernel's (o, lse) against the exact (o64, lse64).

    max_abs_o / max_abs_lse: max |o - O|, max |lse - LSE| over finite LSE;
    floor: max |rn(O) - O|, what rounding the exact output once costs;
    ulps: max |o - rn(O)| in spacings of the output grid at the largest
    |rn(O)| of the element's row (0 for a kernel whose only error is that one
    rounding; the row's scale, since an element near zero has a grid far
    finer than the row's accumulation error); worst: index and values of the
    element with the largest |o - O|.
    """
    o, lse, o64, lse64 = _f64(o), _f64(lse), _f64(o64), _f64(lse64)
    rn = round_to(o64, dtype)
    row_scale = np.abs(rn).max(axis=-1, keepdims=True) if rn.size else rn
    d = np.abs(o - o64)
    fin = np.isfinite(lse64)
    at = np.unravel_index(int(np.argmax(d)), d.shape) if d.size else ()
    return {
        "max_abs_o": float(d.max()) if d.size else 0.0,
        "max_abs_lse": float(np.abs(lse[fin] - lse64[fin]).max()) if fin.any() else 0.0,
        "floor": float(np.abs(rn - o64).max()) if o64.size else 0.0,
        "ulps": float((np.abs(o - rn) / output_ulp(row_scale, dtype)).max()) if o64.size else 0.0,
        "worst": {"index": [int(i) for i in at], "o": float(o[at]) if d.size else 0.0,
                  "o_exact": float(o64[at]) if d.size else 0.0},
    }


__all__ = [
    "attention", "attention_rows", "attention_incremental", "split_partials",
    "split_bounds", "lse_merge", "rope_rotate", "visible_mask", "query_positions",
    "softmax_probs", "rounding_floor", "round_to", "output_ulp", "error_report", "alibi_bias",
]
