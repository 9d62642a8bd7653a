"""Pins for the fp64 oracle, against things other than itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped max
shift, a wrong sign or index in RoPE, a transposed operand, an off-by-one in
the window, a wrong GQA head map, a wrong merge weight) fails at least one test:
  * pure-Python brute force with the textbook (unshifted) softmax;
  * hand-worked cases in tests/golden/hand_cases.json;
  * closed forms (one key, zero scores, constant V, W=1, W >= Nk);
  * invariants (rows of P sum to 1, incremental == three-pass for any tiling
    and tile order, split+merge == unsplit, tree merge == flat merge, shift
    invariance of safe softmax, RoPE relative-position property);
  * a library routine the definition reduces to without RoPE (torch's
    scaled_dot_product_attention in float64 on the CPU, and logsumexp).
"""
import json
import math
import zlib
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import cascade as A
from oracle.brute import brute_attention

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def close(a, b, rtol=1e-12, atol=1e-12):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), "different infinities"
    assert np.array_equal(a[~fin], b[~fin])
    np.testing.assert_allclose(a[fin], b[fin], rtol=rtol, atol=atol)


CASES = [
    # (B, Hq, Hkv, Nq, Nk, D, mask, window, rope_base)
    (1, 1, 1, 6, 6, 4, "none", 0, 0.0),
    (2, 2, 2, 5, 5, 8, "causal", 0, 0.0),
    (1, 4, 2, 7, 9, 4, "causal", 0, 0.0),      # Nq < Nk, GQA 4:2
    (1, 2, 1, 9, 6, 4, "causal", 0, 0.0),      # Nq > Nk: leading rows see nothing
    (1, 2, 2, 8, 8, 4, "sliding", 1, 0.0),
    (2, 1, 1, 9, 9, 6, "sliding", 3, 0.0),
    (1, 4, 2, 5, 11, 4, "sliding", 4, 0.0),
    (1, 1, 1, 6, 6, 8, "none", 0, 10000.0),
    (1, 2, 2, 7, 7, 4, "causal", 0, 10000.0),
    (1, 4, 2, 6, 10, 8, "causal", 0, 100.0),
    (1, 2, 1, 9, 9, 4, "sliding", 3, 500.0),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,D,mask,window,base", CASES)
def test_three_pass_matches_brute_force(B, Hq, Hkv, Nq, Nk, D, mask, window, base):
    seed = zlib.crc32(repr((B, Hq, Hkv, Nq, Nk, D, mask, window, base)).encode())
    q, k, v = rnd((B, Hq, Nq, D), seed), rnd((B, Hkv, Nk, D), seed + 1), rnd((B, Hkv, Nk, D), seed + 2)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, scale, mask, window, base)
    ob, lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, mask, window, base)
    close(o, ob)
    close(lse, lb)
    # the same rows one at a time
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Nq)]
    orow, lrow = oracle.attention_rows(q, k, v, scale, rows, mask, window, base)
    close(orow, o.reshape(-1, D))
    close(lrow, lse.reshape(-1))


def test_hand_cases():
    g = json.load(open(GOLD))
    for c in g["attention"]:
        o, lse = oracle.attention(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                  c["scale"], c["mask"], c["window"], c["rope_base"])
        close(o, c["o"], rtol=1e-14, atol=1e-14)
        close(lse, c["lse"], rtol=1e-14, atol=1e-14)
    for c in g["rope"]:
        out = oracle.rope_rotate(np.array([c["x"]]), np.array([c["pos"]]), c["base"])
        close(out[0], c["out"], rtol=1e-14, atol=1e-15)
    for c in g["merge"]:
        lp = np.array([float(x) for x in c["lse_parts"]])
        o, lse = oracle.lse_merge(np.array(c["o_parts"]), lp)
        close(o, c["o"], rtol=1e-14, atol=1e-15)
        close(lse, c["lse"], rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("mask,window,base", [("none", 0, 0.0), ("causal", 0, 0.0),
                                              ("sliding", 5, 0.0), ("causal", 0, 10000.0)])
def test_rows_of_p_sum_to_one(mask, window, base):
    q, k = rnd((1, 2, 33, 8), 3), rnd((1, 2, 40, 8), 4)
    for h in range(2):
        P = oracle.softmax_probs(q, k, 0.3, mask, window, base, b=0, h=h)
        vis = A.visible_mask(A.query_positions(33, 40), np.arange(40), mask, window)
        assert np.all(P[~vis] == 0.0)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask,window,base", [("none", 0, 0.0), ("causal", 0, 0.0),
                                              ("sliding", 7, 0.0), ("causal", 0, 10000.0),
                                              ("sliding", 20, 10000.0)])
@pytest.mark.parametrize("tile", [1, 3, 64, 128, 150])
def test_incremental_equals_three_pass(mask, window, base, tile):
    q, k, v = rnd((1, 2, 150, 8), 10), rnd((1, 1, 150, 8), 11), rnd((1, 1, 150, 8), 12)
    o, lse = oracle.attention(q, k, v, 0.35, mask, window, base)
    oi, li = oracle.attention_incremental(q, k, v, 0.35, mask, window, base, tile=tile)
    close(oi, o)
    close(li, lse)


def test_incremental_is_order_independent():
    q, k, v = rnd((1, 1, 70, 8), 20), rnd((1, 1, 130, 8), 21), rnd((1, 1, 130, 8), 22)
    o, lse = oracle.attention(q, k, v, 0.5, "causal")
    ntiles = -(-130 // 16)
    for seed in range(3):
        order = np.random.default_rng(seed).permutation(ntiles)
        oi, li = oracle.attention_incremental(q, k, v, 0.5, "causal", tile=16, order=order)
        close(oi, o)
        close(li, lse)


@pytest.mark.parametrize("S", [1, 2, 7, 64])
@pytest.mark.parametrize("mask,window,base", [("none", 0, 0.0), ("causal", 0, 0.0),
                                              ("sliding", 9, 10000.0)])
def test_split_merge_equals_unsplit(S, mask, window, base):
    q, k, v = rnd((2, 4, 3, 8), 30), rnd((2, 2, 100, 8), 31), rnd((2, 2, 100, 8), 32)
    o, lse = oracle.attention(q, k, v, 0.4, mask, window, base)
    op, lp = oracle.split_partials(q, k, v, 0.4, S, mask, window, base)
    om, lm = oracle.lse_merge(op, lp)
    close(om, o)
    close(lm, lse)


def test_tree_merge_equals_flat_merge():
    op, lp = rnd((5, 16, 6), 40), rnd((5, 16), 41, 3.0)
    lp[1, 3] = -np.inf
    of, lf = oracle.lse_merge(op, lp)
    oa, la = oracle.lse_merge(op[:, :5], lp[:, :5])
    ob, lb = oracle.lse_merge(op[:, 5:11], lp[:, 5:11])
    oc, lc = oracle.lse_merge(op[:, 11:], lp[:, 11:])
    ot, lt = oracle.lse_merge(np.stack([oa, ob, oc], axis=1), np.stack([la, lb, lc], axis=1))
    close(ot, of)
    close(lt, lf)


def test_split_bounds_cover_keys_once():
    for Nk, S in [(32768, 64), (100, 7), (5, 8), (1, 1)]:
        b = A.split_bounds(Nk, S)
        covered = [j for lo, hi in b for j in range(lo, hi)]
        assert covered == list(range(Nk))
        if Nk == 32768:
            assert all(hi - lo == 512 for lo, hi in b)


@pytest.mark.parametrize("Nk,S,bounds", [
    # chunk c covers [c*ceil(Nk/S), min(Nk, (c+1)*ceil(Nk/S))), worked by hand:
    # ceil(100/7) = 15, so six full chunks and a short last one [90, 100)
    (100, 7, [(0, 15), (15, 30), (30, 45), (45, 60), (60, 75), (75, 90), (90, 100)]),
    # ceil(5/8) = 1: one key per chunk, the last three chunks empty
    (5, 8, [(0, 1), (1, 2), (2, 3), (3, 4), (4, 5), (5, 5), (6, 6), (7, 7)]),
    # ceil(10/4) = 3: a floor split (2, 2, 3, 3 or 3, 3, 2, 2) would differ
    (10, 4, [(0, 3), (3, 6), (6, 9), (9, 10)]),
    # ceil(7/3) = 3, and a chunk that starts exactly at Nk
    (6, 4, [(0, 2), (2, 4), (4, 6), (6, 6)]),
    (1, 3, [(0, 1), (1, 1), (2, 2)]),
])
def test_split_bounds_hand_cases(Nk, S, bounds):
    # compared as the keys each chunk holds (an empty chunk may be written
    # [lo, hi) with lo >= hi)
    got = [list(range(lo, hi)) for lo, hi in A.split_bounds(Nk, S)]
    assert got == [list(range(lo, hi)) for lo, hi in bounds]
    assert [lo for lo, _ in A.split_bounds(Nk, S)] == [lo for lo, _ in bounds]


# ------------------------------------------------- output rounding and ulps
F16_CASES = [
    # (exact value, its fp16 rounding worked by hand with ties to even)
    (1.0 + 2.0 ** -12, 1.0),                      # grid 2^-10 on [1, 2): a quarter spacing rounds down
    (1.0 + 3 * 2.0 ** -12, 1.0 + 2.0 ** -10),     # nearest is 1+2^-10 (distance 2^-12)
    (1.0 + 2.0 ** -11, 1.0),                      # exact tie between 1 and 1+2^-10 -> even 1.0
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2 * 2.0 ** -10),  # tie between 1+2^-10 (odd) and 1+2^-9 -> 1+2^-9
    (2049.0, 2048.0),                             # spacing 2 above 2048: tie -> even 2048
    (2051.0, 2052.0),                             # tie between 2050 (odd) and 2052 -> 2052
    (-0.3, -1229 * 2.0 ** -12),                   # 0.3 in [0.25, 0.5): spacing 2^-12, 0.3 = 1228.8 spacings
]


def test_round_to_fp16_hand_cases():
    x = np.array([c[0] for c in F16_CASES])
    assert np.array_equal(A.round_to(x, torch.float16), np.array([c[1] for c in F16_CASES]))


def test_rounding_floor_hand_cases():
    # the floor is the largest |rn(x) - x| over the array
    assert A.rounding_floor(np.array([1.0 + 2.0 ** -12, 0.5, 1.0]), torch.float16) == 2.0 ** -12
    assert A.rounding_floor(np.array([2049.0, 1.0 + 2.0 ** -12]), torch.float16) == 1.0
    # bf16 keeps 8 significand bits: spacing 2^-7 on [1, 2); 1 + 2^-8 is a tie -> 1.0
    assert A.rounding_floor(np.array([1.0 + 2.0 ** -8]), torch.bfloat16) == 2.0 ** -8
    assert A.rounding_floor(np.array([3.0 + 2.0 ** -9]), torch.bfloat16) == 2.0 ** -9  # spacing 2^-6 on [2, 4)
    assert A.rounding_floor(np.array([0.25, -4.0, 0.0]), torch.bfloat16) == 0.0        # on the grid
    assert A.rounding_floor(np.zeros(0), torch.float16) == 0.0


def test_output_ulp_matches_library_spacing():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(2000) * 4.0, [1.0, 2.0, 0.75, 2048.0, 2.0 ** -20, 2.0 ** -14, 6e4]])
    h = v.astype(np.float16)
    assert np.array_equal(A.output_ulp(h.astype(np.float64), torch.float16), np.spacing(np.abs(h)).astype(np.float64))
    bt = torch.tensor(v, dtype=torch.bfloat16).abs()
    ref = (torch.nextafter(bt, torch.full_like(bt, float("inf"))) - bt).to(torch.float64).numpy()
    assert np.array_equal(A.output_ulp(bt.to(torch.float64).numpy(), torch.bfloat16), ref)
    f = v.astype(np.float32)
    assert np.array_equal(A.output_ulp(f.astype(np.float64), torch.float32), np.spacing(np.abs(f)).astype(np.float64))


def test_error_report_hand_case():
    o64 = np.array([[1.0 + 2.0 ** -12, 0.5], [2049.0, -1.0]])
    lse64 = np.array([0.5, -np.inf])
    # a kernel that rounds once is 0 ulps off rn(O); one more spacing is 1 ulp
    o = A.round_to(o64, torch.float16)
    r = A.error_report(o, np.array([0.5 + 1e-4, -np.inf]), o64, lse64, torch.float16)
    assert r["ulps"] == 0.0 and r["floor"] == 1.0 and r["max_abs_o"] == 1.0
    assert r["max_abs_lse"] == pytest.approx(1e-4) and r["worst"]["index"] == [1, 0]
    o[0, 1] = 0.5 + 2.0 ** -10   # one fp16 spacing of the row's largest |O| (1.0) above 0.5
    assert A.error_report(o, lse64, o64, lse64, torch.float16)["ulps"] == 1.0
    # an element near zero is measured on its row's scale, not its own grid
    o64 = np.array([[2.0 ** -20, 1.0]])
    o = A.round_to(o64, torch.float16)
    o[0, 0] += 2.0 ** -12        # a quarter spacing at 1.0, 2^12 spacings at 2^-20
    assert A.error_report(o, np.zeros(1), o64, np.zeros(1), torch.float16)["ulps"] == 0.25


# ---------------------------------------------------------------- closed forms
def test_single_key():
    q, k, v = rnd((1, 2, 4, 8), 50), rnd((1, 2, 1, 8), 51), rnd((1, 2, 1, 8), 52)
    o, lse = oracle.attention(q, k, v, 0.7)
    close(o, np.broadcast_to(v, o.shape))
    s = 0.7 * np.einsum("bhid,bhjd->bhij", q, k)[..., 0]
    close(lse, s)


def test_causal_row_zero_sees_only_key_zero():
    q, k, v = rnd((1, 1, 6, 4), 53), rnd((1, 1, 6, 4), 54), rnd((1, 1, 6, 4), 55)
    o, lse = oracle.attention(q, k, v, 1.0, "causal")
    close(o[0, 0, 0], v[0, 0, 0])
    close(lse[0, 0, 0], float(q[0, 0, 0] @ k[0, 0, 0]))


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 3)])
def test_zero_scores_average_visible_values(mask, window):
    q, k, v = rnd((1, 1, 9, 4), 56), rnd((1, 1, 9, 4), 57), rnd((1, 1, 9, 4), 58)
    for qq, sc in [(np.zeros_like(q), 1.0), (q, 0.0)]:
        o, lse = oracle.attention(qq, k, v, sc, mask, window)
        vis = A.visible_mask(np.arange(9), np.arange(9), mask, window)
        for i in range(9):
            close(o[0, 0, i], v[0, 0, vis[i]].mean(axis=0))
            close(lse[0, 0, i], math.log(vis[i].sum()))


def test_constant_values_give_constant_output():
    q, k = rnd((1, 2, 12, 8), 59), rnd((1, 2, 12, 8), 60)
    o, _ = oracle.attention(q, k, np.ones((1, 2, 12, 8)), 0.9, "sliding", window=4, rope_base=10000.0)
    close(o, np.ones_like(o))


def test_window_one_is_diagonal_and_wide_window_is_causal():
    q, k, v = rnd((1, 1, 10, 4), 61), rnd((1, 1, 10, 4), 62), rnd((1, 1, 10, 4), 63)
    o1, _ = oracle.attention(q, k, v, 1.0, "sliding", window=1)
    close(o1, v)
    ow, lw = oracle.attention(q, k, v, 1.0, "sliding", window=10)
    oc, lc = oracle.attention(q, k, v, 1.0, "causal")
    close(ow, oc)
    close(lw, lc)


def test_fully_masked_rows_are_zero_with_neg_inf_lse():
    q, k, v = rnd((1, 1, 6, 4), 64), rnd((1, 1, 3, 4), 65), rnd((1, 1, 3, 4), 66)
    o, lse = oracle.attention(q, k, v, 1.0, "causal")   # p_i = i - 3
    assert np.all(o[0, 0, :3] == 0) and np.all(lse[0, 0, :3] == -np.inf)
    assert np.all(np.isfinite(lse[0, 0, 3:]))


def test_safe_softmax_survives_huge_scores():
    """Append one dimension carrying a constant c: every score of a row moves by c*scale.

    O must not change and LSE moves by exactly c*scale, with c large enough
    that an unshifted exp would overflow to inf.
    """
    q, k, v = rnd((1, 1, 8, 4), 67), rnd((1, 1, 8, 4), 68), rnd((1, 1, 8, 4), 69)
    o, lse = oracle.attention(q, k, v, 0.5, "causal")
    c = 4000.0
    qe = np.concatenate([q, np.full((1, 1, 8, 1), c)], axis=-1)
    ke = np.concatenate([k, np.ones((1, 1, 8, 1))], axis=-1)
    ve = np.concatenate([v, np.zeros((1, 1, 8, 1))], axis=-1)
    o2, lse2 = oracle.attention(qe, ke, ve, 0.5, "causal")
    close(o2[..., :4], o, rtol=1e-9, atol=1e-12)
    close(lse2 - 0.5 * c, lse, rtol=0, atol=1e-9)


# ---------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity_and_norm_preserved():
    x = rnd((1, 5, 16), 70)
    close(oracle.rope_rotate(x[:, :1], np.array([0]), 10000.0), x[:, :1], rtol=0, atol=0)
    r = oracle.rope_rotate(x, np.arange(5) * 37, 10000.0)
    n_in = x[..., :8] ** 2 + x[..., 8:] ** 2
    n_out = r[..., :8] ** 2 + r[..., 8:] ** 2
    close(n_out, n_in)


def test_rope_d2_is_plane_rotation():
    for pos in [0, 1, 5, 1234]:
        r = oracle.rope_rotate(np.array([[1.0, 0.0], [0.0, 1.0]]), np.array([pos, pos]), 10000.0)
        close(r, [[math.cos(pos), math.sin(pos)], [-math.sin(pos), math.cos(pos)]], atol=1e-15)


def test_rope_scores_depend_only_on_relative_position():
    q, k = rnd((1, 16), 71), rnd((1, 16), 72)
    for base in [10000.0, 50.0]:
        s = []
        for shift in [0, 3, 1000]:
            qr = oracle.rope_rotate(q, np.array([7 + shift]), base)
            kr = oracle.rope_rotate(k, np.array([2 + shift]), base)
            s.append(float(qr[0] @ kr[0]))
        np.testing.assert_allclose(s, s[0], rtol=1e-12)


# ---------------------------------------------------------------- GQA
def test_gqa_equals_mha_on_repeated_kv():
    q, k, v = rnd((2, 8, 5, 8), 80), rnd((2, 2, 9, 8), 81), rnd((2, 2, 9, 8), 82)
    o, lse = oracle.attention(q, k, v, 0.3, "causal", rope_base=10000.0)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    o2, lse2 = oracle.attention(q, kr, vr, 0.3, "causal", rope_base=10000.0)
    close(o, o2)
    close(lse, lse2)


# ---------------------------------------------------------------- library routine
@pytest.mark.parametrize("mask,window,Nq,Nk", [("none", 0, 17, 23), ("causal", 0, 31, 31),
                                               ("causal", 0, 9, 20), ("sliding", 6, 25, 25)])
def test_matches_torch_sdpa_float64(mask, window, Nq, Nk):
    q, k, v = rnd((2, 3, Nq, 16), 90), rnd((2, 3, Nk, 16), 91), rnd((2, 3, Nk, 16), 92)
    scale = 0.21
    o, lse = oracle.attention(q, k, v, scale, mask, window)
    vis = A.visible_mask(A.query_positions(Nq, Nk), np.arange(Nk), mask, window)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    tm = torch.from_numpy(vis)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale)
    s = (tq @ tk.transpose(-1, -2)) * scale
    ref_lse = torch.logsumexp(s.masked_fill(~tm, -math.inf), dim=-1)
    close(o, ref.numpy(), rtol=1e-11, atol=1e-13)
    close(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-13)


def test_oracle_consumes_low_precision_inputs_exactly():
    from workloads import gen_qkv
    q, k, v = gen_qkv(1, 2, 2, 16, 16, 8, "bf16", seed=7)
    o1, l1 = oracle.attention(q, k, v, 0.25, "causal")
    o2, l2 = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.25, "causal")
    close(o1, o2, rtol=0, atol=0)
    close(l1, l2, rtol=0, atol=0)


# ---------------------------------------------------------------- ALiBi
ALIBI_CASES = [
    (1, 2, 2, 7, 7, 4, "causal", 0, 0.0),
    (1, 4, 2, 6, 9, 4, "none", 0, 0.0),
    (1, 2, 1, 8, 8, 4, "sliding", 3, 10000.0),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,D,mask,window,base", ALIBI_CASES)
def test_alibi_matches_brute_force(B, Hq, Hkv, Nq, Nk, D, mask, window, base):
    from workloads import alibi_slopes
    seed = zlib.crc32(repr(("alibi", B, Hq, Nq, Nk, mask)).encode())
    q, k, v = rnd((B, Hq, Nq, D), seed), rnd((B, Hkv, Nk, D), seed + 1), rnd((B, Hkv, Nk, D), seed + 2)
    sl = alibi_slopes(Hq)
    o, lse = oracle.attention(q, k, v, 0.5, mask, window, base, alibi_slopes=sl)
    ob, lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), 0.5, mask, window, base, alibi_slopes=sl)
    close(o, ob)
    close(lse, lb)
    oi, li = oracle.attention_incremental(q, k, v, 0.5, mask, window, base, tile=3, alibi_slopes=sl)
    close(oi, o)
    close(li, lse)
    op, lp = oracle.split_partials(q, k, v, 0.5, 3, mask, window, base, alibi_slopes=sl)
    om, lm = oracle.lse_merge(op, lp)
    close(om, o)
    close(lm, lse)
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Nq)]
    orow, lrow = oracle.attention_rows(q, k, v, 0.5, rows, mask, window, base, alibi_slopes=sl)
    close(orow, o.reshape(-1, D))
    close(lrow, lse.reshape(-1))


def test_alibi_zero_scores_give_geometric_weights():
    """q = 0: weights exp(-m (p - j)) / sum, a closed form; V = identity picks them out."""
    N, m = 5, 0.7
    q = np.zeros((1, 1, N, N))
    k = rnd((1, 1, N, N), 120)
    v = np.eye(N)[None, None]
    o, lse = oracle.attention(q, k, v, 1.0, "causal", alibi_slopes=[m])
    for i in range(N):
        w = np.array([math.exp(-m * (i - j)) for j in range(i + 1)])
        close(o[0, 0, i, : i + 1], w / w.sum(), rtol=1e-14, atol=1e-15)
        close(o[0, 0, i, i + 1:], np.zeros(N - i - 1), rtol=0, atol=0)
        close(lse[0, 0, i], math.log(w.sum()), rtol=1e-14, atol=1e-15)


def test_alibi_zero_slope_is_plain_attention_and_matches_sdpa():
    q, k, v = rnd((1, 3, 10, 8), 121), rnd((1, 3, 10, 8), 122), rnd((1, 3, 10, 8), 123)
    o0, l0 = oracle.attention(q, k, v, 0.3, "causal")
    o1, l1 = oracle.attention(q, k, v, 0.3, "causal", alibi_slopes=[0.0, 0.0, 0.0])
    close(o1, o0)
    close(l1, l0)
    sl = [0.5, 0.25, 0.125]
    o2, _ = oracle.attention(q, k, v, 0.3, "causal", alibi_slopes=sl)
    pos = np.arange(10)
    bias = np.stack([A.alibi_bias(s, pos, pos) for s in sl])[None]
    vis = A.visible_mask(pos, pos, "causal")
    mask = torch.from_numpy(np.where(vis, bias, -np.inf))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=0.3)
    close(o2, ref.numpy(), rtol=1e-11, atol=1e-13)


# ------------------------------------------- whole-output report (oracle/report.py)
def test_compare_full_reports_rounding_only_and_finds_a_planted_error():
    from oracle import report
    q, k, v = (t for t in __import__("workloads").gen_qkv(2, 4, 2, 40, 40, 8, torch.float16, 21))
    o64, l64 = oracle.attention(q, k, v, 0.3, "causal")
    o = torch.from_numpy(o64).to(torch.float16)         # the exact result rounded once
    lse = torch.from_numpy(l64).to(torch.float32)
    r = report.compare_full(q, k, v, o, lse, 0.3, "causal", 0, 0.0, torch.float16)
    assert r["ulps"] == 0.0 and r["max_abs_o"] == r["floor"] > 0
    assert r["max_abs_lse"] < 1e-6
    o[1, 3, 17, 5] += 0.25                              # one wrong element in head 3 (KV group 1)
    lse[0, 2, 9] = 7.0
    r = report.compare_full(q, k, v, o, lse, 0.3, "causal", 0, 0.0, torch.float16)
    assert r["worst"]["index"] == [1, 3, 17, 5] and r["max_abs_o"] > 0.2
    assert r["max_abs_lse"] == pytest.approx(abs(7.0 - l64[0, 2, 9]), rel=1e-6)
    lse[0, 2, 9] = -float("inf")                        # a -inf where a key is visible
    assert report.compare_full(q, k, v, o, lse, 0.3, "causal", 0, 0.0, torch.float16)["max_abs_lse"] == float("inf")


def test_compare_partials_against_merge():
    from oracle import report
    q, k, v = (t for t in __import__("workloads").gen_qkv(1, 4, 2, 1, 50, 8, torch.float32, 22))
    op, lp = oracle.split_partials(q, k, v, 0.5, 4)
    assert report.compare_partials(q, k, v, torch.from_numpy(op), torch.from_numpy(lp), 0.5, 4) == (0.0, 0.0)
    op[0, 1, 0, 2, 3] += 1e-3
    e_o, e_l = report.compare_partials(q, k, v, torch.from_numpy(op), torch.from_numpy(lp), 0.5, 4)
    assert e_o == pytest.approx(1e-3) and e_l == 0.0
