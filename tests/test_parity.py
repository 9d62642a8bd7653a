"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (max-abs over every output element, O and LSE alike): 2e-3 for
fp16 and fp32, 1e-2 for bf16, as stated for the method's fp16/bf16 outputs
with fp32 accumulation; fp32 inputs reuse the strictest stated bound.  LSE is
compared element by element in its [B, Hq, Nq] layout, with the positions of
-inf (rows that see no key) required to match exactly.  Outputs are poisoned
with NaN before each launch so an unwritten element fails.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import attention_pass_cascaded_amd as rf
import oracle
from workloads import gen_qkv

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-3, "f16": 2e-3, "bf16": 1e-2}
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def compare(o, lse, ref_o, ref_lse, tol, what=""):
    o = o.detach().float().cpu().double().numpy()
    lse = lse.detach().cpu().double().numpy()
    assert o.shape == ref_o.shape and lse.shape == ref_lse.shape
    assert np.all(np.isfinite(o)), f"{what}: non-finite output element"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf rows differ"
    assert np.all(lse[~fin] == -np.inf)
    err_o = float(np.abs(o - ref_o).max()) if o.size else 0.0
    err_l = float(np.abs(lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    assert err_o <= tol, f"{what}: max |O - O_ref| = {err_o:.3e} > {tol}"
    assert err_l <= tol, f"{what}: max |LSE - LSE_ref| = {err_l:.3e} > {tol}"
    return err_o, err_l


def run_fwd(q, k, v, scale, mask, window, rope):
    dev = torch.device("cuda")
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    out = torch.full_like(qg, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=dev)
    o, l = rf.fwd(qg, kg, vg, scale=scale, mask=mask, window=window, rope_base=rope, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, l


FWD_CASES = [
    # dtype, D, B, Hq, Hkv, Nq, Nk, mask, window, rope
    ("f16", 64, 1, 2, 2, 129, 129, "none", 0, 0.0),
    ("f16", 64, 2, 3, 3, 300, 300, "causal", 0, 0.0),
    ("f16", 64, 1, 4, 2, 70, 300, "causal", 0, 0.0),
    ("f16", 64, 1, 2, 1, 150, 100, "causal", 0, 0.0),
    ("f16", 64, 1, 2, 2, 1, 1, "causal", 0, 0.0),
    ("f16", 64, 1, 2, 2, 17, 17, "none", 0, 0.0),
    ("f16", 64, 1, 2, 2, 257, 257, "causal", 0, 10000.0),
    ("f16", 64, 1, 2, 2, 200, 333, "sliding", 37, 10000.0),
    ("f16", 128, 1, 2, 2, 300, 300, "sliding", 64, 0.0),
    ("bf16", 128, 1, 2, 2, 520, 520, "sliding", 256, 0.0),
    ("bf16", 128, 2, 2, 2, 131, 131, "sliding", 1, 0.0),
    ("bf16", 128, 1, 4, 1, 200, 200, "causal", 0, 10000.0),
    ("bf16", 64, 1, 2, 2, 190, 190, "none", 0, 500.0),
    ("bf16", 128, 1, 2, 2, 64, 64, "none", 0, 0.0),
    # D = 128 16-bit without RoPE: direct-to-LDS K/V, single V buffer; GQA,
    # Nq < Nk with bottom-right alignment and ragged tails
    ("bf16", 128, 2, 4, 2, 190, 333, "causal", 0, 0.0),
    ("f16", 128, 1, 4, 1, 77, 77, "none", 0, 0.0),
    ("bf16", 128, 1, 2, 2, 129, 700, "sliding", 200, 0.0),
    ("f16", 128, 1, 2, 1, 150, 100, "causal", 0, 0.0),      # Nq > Nk: the first 50 rows see no key
    # D = 128 16-bit sliding window: tiles visited in cyclic order from a
    # grid-aligned start, with windows that are not tile multiples
    ("f16", 128, 1, 2, 2, 777, 777, "sliding", 300, 0.0),
    ("bf16", 128, 1, 3, 1, 400, 1000, "sliding", 97, 0.0),
    ("f16", 128, 1, 2, 2, 1, 300, "sliding", 50, 0.0),       # one query row at position 299
    ("bf16", 128, 1, 2, 1, 200, 200, "sliding", 5000, 0.0),  # window wider than the sequence
    # RoPE over many tiles and at large positions (up to 70,000 keys, so
    # angles of thousands of revolutions), with windows starting mid-tile
    ("f16", 64, 1, 2, 2, 64, 2100, "causal", 0, 10000.0),
    ("bf16", 64, 1, 2, 1, 40, 1500, "none", 0, 10000.0),
    ("f16", 64, 1, 2, 2, 100, 1400, "sliding", 1200, 10000.0),
    ("f16", 64, 1, 1, 1, 16, 70000, "causal", 0, 10000.0),
    # D = 128 RoPE: each thread rotates two rows of a K tile; long enough key
    # ranges that the carried angle passes several exact re-anchors
    ("f16", 128, 1, 2, 1, 130, 3000, "causal", 0, 10000.0),
    ("bf16", 128, 1, 2, 2, 200, 5000, "sliding", 700, 500000.0),
    ("f32", 128, 1, 1, 1, 50, 4500, "causal", 0, 10000.0),
    ("f32", 64, 1, 1, 1, 256, 256, "none", 0, 0.0),
    ("f32", 64, 1, 2, 2, 100, 100, "causal", 0, 10000.0),
    ("f32", 128, 1, 2, 1, 77, 150, "sliding", 40, 0.0),
]


@pytest.mark.parametrize("dt,D,B,Hq,Hkv,Nq,Nk,mask,window,rope", FWD_CASES)
def test_fwd_matches_oracle(dt, D, B, Hq, Hkv, Nq, Nk, mask, window, rope):
    seed = zlib.crc32(repr((dt, D, B, Hq, Hkv, Nq, Nk, mask, window, rope)).encode()) % 10_000
    q, k, v = gen_qkv(B, Hq, Hkv, Nq, Nk, D, dt, seed)
    scale = 1.0 / math.sqrt(D)
    print(f"case fwd {dt} D={D} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} {mask} W={window} rope={rope}", flush=True)
    o, lse = run_fwd(q, k, v, scale, mask, window, rope)
    ro, rl = oracle.attention(q, k, v, scale, mask, window, rope)
    compare(o, lse, ro, rl, TOL[dt], "fwd")


# 16-bit D = 64 forwards run as 128-row work-groups of 4 waves (layout 0) or,
# when the grid is small, with the key range cut in two halves that two groups
# of waves run and merge in LDS: 64-row work-groups of two wave pairs
# (layout 1) or 128-row work-groups of two 4-wave groups (layout 2);
# RF_ATTN_KEY_HALVES forces a layout.
# Every D = 64 16-bit case runs all three ways, plus cases aimed at the halves:
# odd tile counts (the second half one tile short), a single tile (the second
# half empty, so the merge takes -inf from it), rows that see no key.
D64_CASES = [c for c in FWD_CASES if c[1] == 64 and c[0] != "f32"] + [
    ("f16", 64, 1, 2, 2, 64, 96, "none", 0, 0.0),        # 3 tiles of 32 keys
    ("bf16", 64, 1, 2, 2, 40, 20, "none", 0, 0.0),       # one tile
    ("f16", 64, 1, 3, 1, 200, 120, "causal", 0, 0.0),    # first 80 rows see no key
    ("bf16", 64, 2, 4, 2, 333, 900, "sliding", 100, 10000.0),
    ("f16", 64, 1, 2, 2, 70, 4100, "none", 0, 10000.0),  # 129 tiles: re-anchor inside each half
]


@pytest.mark.parametrize("halves", ["0", "1", "2"])
@pytest.mark.parametrize("dt,D,B,Hq,Hkv,Nq,Nk,mask,window,rope", D64_CASES)
def test_fwd_d64_both_layouts(monkeypatch, halves, dt, D, B, Hq, Hkv, Nq, Nk, mask, window, rope):
    monkeypatch.setenv("RF_ATTN_KEY_HALVES", halves)
    seed = zlib.crc32(repr((dt, D, B, Hq, Hkv, Nq, Nk, mask, window, rope)).encode()) % 10_000
    q, k, v = gen_qkv(B, Hq, Hkv, Nq, Nk, D, dt, seed)
    scale = 1.0 / math.sqrt(D)
    print(f"case fwd halves={halves} {dt} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} {mask} W={window} rope={rope}", flush=True)
    o, lse = run_fwd(q, k, v, scale, mask, window, rope)
    ro, rl = oracle.attention(q, k, v, scale, mask, window, rope)
    compare(o, lse, ro, rl, TOL[dt], f"fwd halves={halves}")


@pytest.mark.parametrize("halves", ["0", "1", "2"])
def test_fwd_d64_alibi_both_layouts(monkeypatch, halves):
    from workloads import alibi_slopes
    monkeypatch.setenv("RF_ATTN_KEY_HALVES", halves)
    q, k, v = gen_qkv(1, 4, 2, 150, 400, 64, "f16", 77)
    sl = alibi_slopes(4)
    print(f"case alibi fwd halves={halves}", flush=True)
    for mask, rope in (("causal", 0.0), ("none", 10000.0)):
        dev = torch.device("cuda")
        o, lse = rf.fwd(q.to(dev), k.to(dev), v.to(dev), scale=0.125, mask=mask, rope_base=rope, alibi_slopes=sl)
        torch.cuda.synchronize()
        ro, rl = oracle.attention(q, k, v, 0.125, mask, 0, rope, alibi_slopes=sl)
        compare(o, lse, ro, rl, TOL["f16"], f"alibi halves={halves} {mask}")


@pytest.mark.parametrize("scale", [0.125, 0.69, 0.7, 1.0, 4.0])
def test_fwd_f16_d64_scale_range_matches_oracle(scale):
    """fp16, D = 64, no RoPE or ALiBi, over a range of scales with Q tripled
    so the weights are far from uniform: larger scores must not cost
    accuracy (the scores are formed from the unscaled fp16 q and k, and the
    scale is applied in fp32)."""
    q, k, v = gen_qkv(1, 3, 3, 300, 300, 64, "f16", 5)
    q = (q.float() * 3).half()
    print(f"case fwd f16 D=64 scale={scale}", flush=True)
    for mask in ("causal", "none"):
        o, lse = run_fwd(q, k, v, scale, mask, 0, 0.0)
        ro, rl = oracle.attention(q, k, v, scale, mask)
        compare(o, lse, ro, rl, TOL["f16"], f"scale {scale} {mask}")


@pytest.mark.parametrize("mask", ["causal", "none"])
def test_fwd_f16_d64_late_dominant_key(mask):
    """fp16, D = 64: keys far past the first tile whose scores exceed every
    earlier one by more than 2^16 in the terms (rows of one head only), so the
    reference taken from a row's first tile no longer holds and the block must
    be redone with the running max; the result must still match the oracle."""
    q, k, v = gen_qkv(1, 2, 2, 700, 700, 64, "f16", 6)
    q = q.float()
    k = k.float()
    q[0, 1] = q[0, 1].abs() + 0.5                      # head 1: positive queries
    k[0, 1, 300] = 4.0                                  # dominant keys at 300 and 650
    k[0, 1, 650] = 3.0
    q, k = q.half(), k.half()
    print(f"case fwd f16 D=64 dominant late keys {mask}", flush=True)
    o, lse = run_fwd(q, k, v, 0.125, mask, 0, 0.0)
    ro, rl = oracle.attention(q, k, v, 0.125, mask)
    compare(o, lse, ro, rl, TOL["f16"], f"late dominant key {mask}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_fwd_d128_sliding_dominant_keys(dt):
    """D = 128 sliding window: a dominant key inside each row's window, at
    different offsets from the tile the work-group visits first, so the
    running max must move mid-row whatever the visiting order."""
    q, k, v = gen_qkv(1, 2, 2, 600, 600, 128, dt, 8)
    q = q.float()
    k = k.float()
    q[0, 1] = q[0, 1].abs() + 0.5
    for j in (100, 230, 390, 520):
        k[0, 1, j] = 3.0
    q, k = q.to(v.dtype), k.to(v.dtype)
    print(f"case fwd {dt} D=128 sliding dominant keys", flush=True)
    o, lse = run_fwd(q, k, v, 1 / math.sqrt(128), "sliding", 200, 0.0)
    ro, rl = oracle.attention(q, k, v, 1 / math.sqrt(128), "sliding", 200)
    compare(o, lse, ro, rl, TOL[dt], f"sliding dominant keys {dt}")


def test_fwd_empty_keys_gives_zero_and_neg_inf():
    q, k, v = gen_qkv(1, 2, 2, 40, 0, 64, "f16", 1)
    o, lse = run_fwd(q, k, v, 0.125, "none", 0, 0.0)
    assert torch.all(o == 0) and torch.all(lse == -math.inf)


def test_fwd_scale_zero_averages_values():
    q, k, v = gen_qkv(1, 1, 1, 50, 90, 64, "f32", 2)
    o, lse = run_fwd(q, k, v, 0.0, "causal", 0, 0.0)
    ro, rl = oracle.attention(q, k, v, 0.0, "causal")
    compare(o, lse, ro, rl, 1e-5, "scale 0")


def test_fwd_is_deterministic():
    q, k, v = gen_qkv(1, 2, 2, 300, 300, 64, "f16", 3)
    o1, l1 = run_fwd(q, k, v, 0.125, "causal", 0, 10000.0)
    o2, l2 = run_fwd(q, k, v, 0.125, "causal", 0, 10000.0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_runs_on_the_callers_stream():
    q, k, v = (t.cuda() for t in gen_qkv(1, 2, 2, 256, 256, 64, "f16", 4))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = rf.fwd(q, k, v, scale=0.125, mask="causal")
    s.synchronize()
    ro, rl = oracle.attention(q.cpu(), k.cpu(), v.cpu(), 0.125, "causal")
    compare(o, lse, ro, rl, TOL["f16"], "stream")


SPLIT_CASES = [
    # dtype, D, B, Hq, Hkv, Nq, Nk, S, mask, window, rope     (rows = Hq/Hkv*Nq)
    ("bf16", 128, 2, 8, 2, 1, 1000, 7, "none", 0, 0.0),       # decode kernel, 4 rows
    ("bf16", 128, 1, 4, 4, 1, 512, 1, "none", 0, 0.0),        # 1 row, 1 chunk
    ("f16", 64, 1, 8, 1, 1, 700, 64, "none", 0, 0.0),         # 8 rows, chunks of 11
    ("f16", 64, 1, 4, 2, 3, 300, 5, "causal", 0, 0.0),        # 6 rows, causal with Nq < Nk
    ("bf16", 128, 1, 4, 1, 2, 400, 3, "sliding", 100, 10000.0),
    ("f32", 128, 1, 2, 2, 1, 333, 4, "none", 0, 10000.0),
    ("f16", 128, 1, 2, 2, 1, 50, 64, "none", 0, 0.0),         # more chunks than keys/chunk
    ("f16", 64, 1, 2, 2, 40, 300, 3, "causal", 0, 0.0),       # 40 rows: MFMA split path
    ("bf16", 128, 1, 4, 2, 100, 100, 4, "sliding", 30, 10000.0),
    ("bf16", 128, 1, 16, 1, 1, 900, 5, "none", 0, 0.0),       # 16 rows: widest decode group
    ("f16", 64, 2, 8, 2, 4, 777, 6, "causal", 0, 0.0),        # 16 rows, causal, Nq < Nk
    ("f16", 128, 1, 8, 8, 1, 300, 2, "sliding", 50, 10000.0), # 1 row, f16 RoPE
    ("bf16", 64, 1, 12, 4, 2, 260, 3, "causal", 0, 10000.0),  # 6 rows, bf16 RoPE (hi/lo split)
    ("f32", 64, 1, 8, 1, 1, 200, 3, "none", 0, 0.0),          # float32: vector-ALU decode, 8 rows
    ("f32", 128, 1, 9, 1, 1, 200, 3, "none", 0, 0.0),         # float32, 9 rows: MFMA split path
    ("bf16", 128, 1, 17, 1, 1, 300, 2, "none", 0, 0.0),       # 17 rows: MFMA split path
]


@pytest.mark.parametrize("dt,D,B,Hq,Hkv,Nq,Nk,S,mask,window,rope", SPLIT_CASES)
def test_splitkv_and_merge_match_oracle(dt, D, B, Hq, Hkv, Nq, Nk, S, mask, window, rope):
    seed = zlib.crc32(repr((dt, D, B, Hq, Hkv, Nq, Nk, S, mask, window, rope)).encode()) % 10_000
    q, k, v = gen_qkv(B, Hq, Hkv, Nq, Nk, D, dt, seed)
    scale = 1.0 / math.sqrt(D)
    print(f"case split {dt} D={D} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} S={S} {mask} W={window} rope={rope}", flush=True)
    dev = torch.device("cuda")
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    op = torch.full((B, Hq, Nq, S, D), float("nan"), device=dev)
    lp = torch.full((B, Hq, Nq, S), float("nan"), device=dev)
    rf.splitkv_fwd(qg, kg, vg, S, scale, mask, window, rope, o_part=op, lse_part=lp)
    o, lse = rf.lse_merge(op, lp, out_dtype=DT[dt])
    torch.cuda.synchronize()
    rop, rlp = oracle.split_partials(q, k, v, scale, S, mask, window, rope)
    compare(op, lp, rop, rlp, TOL[dt], "partials (fp32)")
    ro, rl = oracle.attention(q, k, v, scale, mask, window, rope)
    compare(o, lse, ro, rl, TOL[dt], "merged")


def test_merge_matches_oracle_with_empty_chunks():
    g = torch.Generator().manual_seed(11)
    op = torch.randn((3, 5, 9, 128), generator=g)
    lp = torch.randn((3, 5, 9), generator=g) * 4
    lp[0, 1, 2] = -math.inf
    lp[2, 3, :] = -math.inf            # a row with every chunk empty
    op[2, 3] = 0.0
    o, lse = rf.lse_merge(op.cuda(), lp.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.lse_merge(op, lp)
    compare(o, lse, ro, rl, 1e-5, "merge")


# ---------------------------------------------------------------- ALiBi (AttnFuse Table 6)
ALIBI_FWD = [
    ("f16", 64, 1, 4, 4, 300, 300, "causal", 0, 0.0),
    ("bf16", 128, 1, 8, 2, 150, 270, "none", 0, 0.0),
    ("f16", 64, 1, 4, 2, 200, 200, "sliding", 60, 10000.0),
    ("f32", 64, 1, 2, 2, 100, 100, "causal", 0, 0.0),
]


@pytest.mark.parametrize("dt,D,B,Hq,Hkv,Nq,Nk,mask,window,rope", ALIBI_FWD)
def test_fwd_alibi_matches_oracle(dt, D, B, Hq, Hkv, Nq, Nk, mask, window, rope):
    from workloads import alibi_slopes
    seed = zlib.crc32(repr(("alibi", dt, D, Hq, Nq, Nk, mask)).encode()) % 10_000
    q, k, v = gen_qkv(B, Hq, Hkv, Nq, Nk, D, dt, seed)
    sl = alibi_slopes(Hq)
    scale = 1.0 / math.sqrt(D)
    print(f"case alibi fwd {dt} D={D} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} {mask} W={window} rope={rope}", flush=True)
    dev = torch.device("cuda")
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), device=dev)
    rf.fwd(q.to(dev), k.to(dev), v.to(dev), scale=scale, mask=mask, window=window, rope_base=rope,
           out=out, lse=lse, alibi_slopes=sl)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, scale, mask, window, rope, alibi_slopes=sl)
    compare(out, lse, ro, rl, TOL[dt], "alibi fwd")


ALIBI_SPLIT = [
    ("bf16", 128, 2, 8, 2, 1, 1000, 7, "none", 0, 0.0),       # matrix-core decode kernel
    ("f16", 64, 1, 8, 2, 2, 500, 4, "causal", 0, 0.0),        # decode kernel, 8 rows, causal
    ("f32", 128, 1, 4, 1, 1, 333, 3, "none", 0, 0.0),         # vector-ALU decode kernel
    ("bf16", 64, 1, 4, 4, 40, 260, 3, "causal", 0, 10000.0),  # forward kernel in split mode
]


@pytest.mark.parametrize("dt,D,B,Hq,Hkv,Nq,Nk,S,mask,window,rope", ALIBI_SPLIT)
def test_splitkv_alibi_matches_oracle(dt, D, B, Hq, Hkv, Nq, Nk, S, mask, window, rope):
    from workloads import alibi_slopes
    seed = zlib.crc32(repr(("alibi-split", dt, D, Hq, Nq, Nk, S, mask)).encode()) % 10_000
    q, k, v = gen_qkv(B, Hq, Hkv, Nq, Nk, D, dt, seed)
    sl = alibi_slopes(Hq)
    scale = 1.0 / math.sqrt(D)
    print(f"case alibi split {dt} D={D} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} S={S} {mask} rope={rope}", flush=True)
    dev = torch.device("cuda")
    o, lse = rf.decode(q.to(dev), k.to(dev), v.to(dev), num_splits=S, scale=scale, mask=mask, window=window,
                       rope_base=rope, alibi_slopes=sl)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, scale, mask, window, rope, alibi_slopes=sl)
    compare(o, lse, ro, rl, TOL[dt], "alibi split")


# ---------------------------------------------------------------- standalone RoPE (Rotation Calculus)
# several (B, H) layouts of the rows (the kernel indexes rows * N positions)
@pytest.mark.parametrize("dt,D,N,pos,BH", [("f16", 64, 77, 0, (2, 3)), ("bf16", 128, 130, 1000, (2, 3)),
                                            ("f32", 64, 33, 5, (2, 3)), ("f16", 128, 1, 32767, (2, 3)),
                                            ("f32", 128, 300, 1 << 20, (2, 3)), ("bf16", 64, 50, 7, (3, 5)),
                                            ("f16", 128, 65, 0, (4, 4))])
def test_rope_rotate_matches_oracle(dt, D, N, pos, BH):
    g = torch.Generator().manual_seed(zlib.crc32(repr(("rope", dt, D, N, pos)).encode()))
    x = torch.randn((*BH, N, D), generator=g).to(DT[dt])
    ref = oracle.rope_rotate(x, np.arange(N) + pos, 10000.0)          # fp64
    y = rf.rope_rotate(x.cuda(), 10000.0, pos_offset=pos)
    xi = x.cuda().clone()
    rf.rope_rotate(xi, 10000.0, pos_offset=pos, out=xi)                 # in place
    torch.cuda.synchronize()
    got = y.float().cpu().double().numpy()
    assert torch.equal(xi, y)
    # one rounding of the exact rotation to the dtype, plus the float32 arithmetic
    # before it, relative to the pair's size |x_i| + |x_partner|: the angle's
    # fraction of a revolution rounded to fp32 (2^-24 rev), the hardware
    # sin/cos, two products and a sum in fp32; 2^-20 covers them with margin
    # (measured at most 2.4e-7 of the pair, positions up to 2^20)
    mant = {"f16": 10, "bf16": 7, "f32": 23}[dt]
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - mant)
    xd = x.double().numpy()
    pair = np.abs(xd[..., :D // 2]) + np.abs(xd[..., D // 2:])
    pair = np.concatenate([pair, pair], axis=-1)
    err = np.abs(got - ref)
    assert np.all(err <= ulp + 2.0 ** -20 * pair), float(((err - ulp) / np.maximum(pair, 1e-30)).max())


@pytest.mark.parametrize("mask,window", [("causal", 0), ("sliding", 100)])
def test_prerotated_path_matches_oracle_and_fused(mask, window):
    q, k, v = gen_qkv(1, 4, 4, 300, 300, 64, "f16", 21)
    dev = torch.device("cuda")
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    o1, l1 = rf.fwd(qg, kg, vg, scale=0.125, mask=mask, window=window, rope_base=10000.0)
    o2, l2 = rf.fwd_prerotated(qg, kg, vg, 10000.0, scale=0.125, mask=mask, window=window)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, 0.125, mask, window, 10000.0)
    compare(o2, l2, ro, rl, TOL["f16"], "prerotated")
    # same fp16 rounding of the rotated operands on both sides: nearly identical
    assert float((o1.float() - o2.float()).abs().max()) <= 2e-3


def test_rope_mode_auto_switches_above_crossover():
    from attention_pass_cascaded_amd._binding import ROPE_FUSED_MAX_N
    N = ROPE_FUSED_MAX_N + 100
    q, k, v = gen_qkv(1, 1, 1, 40, N, 64, "f16", 22)
    dev = torch.device("cuda")
    o, lse = rf.fwd(q.to(dev), k.to(dev), v.to(dev), scale=0.125, mask="causal", rope_base=10000.0,
                    rope_mode="auto")
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, 0.125, "causal", rope_base=10000.0)
    compare(o, lse, ro, rl, TOL["f16"], "auto rope")


# ---------------------------------------------------------------------------
# A caller-provided output buffer of the wrong shape, dtype or layout is
# refused by the binding before any pointer reaches a kernel.
# ---------------------------------------------------------------------------
def _bad_buffer_calls():
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in gen_qkv(1, 4, 2, 8, 40, 64, torch.float16, 11))
    f32 = dict(dtype=torch.float32, device=dev)
    o_part_s3 = torch.empty(1, 4, 8, 3, 64, **f32)
    lse_part_s3 = torch.empty(1, 4, 8, 3, **f32)
    o, lse = rf.fwd(q, k, v, mask="causal")
    dout = torch.randn_like(o)
    x = torch.randn(6, 64, device=dev, dtype=torch.float16)
    gamma, beta = torch.ones(64, device=dev, dtype=torch.float16), torch.zeros(64, device=dev, dtype=torch.float16)
    return [
        ("fwd out dtype", lambda: rf.fwd(q, k, v, out=torch.empty(q.shape, **f32))),
        ("fwd out too small", lambda: rf.fwd(q, k, v, out=torch.empty(1, 4, 7, 64, dtype=q.dtype, device=dev))),
        ("fwd lse dtype", lambda: rf.fwd(q, k, v, lse=torch.empty(1, 4, 8, dtype=torch.float16, device=dev))),
        ("fwd out transposed", lambda: rf.fwd(q, k, v, out=torch.empty(1, 4, 64, 8, dtype=q.dtype, device=dev).transpose(2, 3))),
        ("split o_part for 3 chunks", lambda: rf.splitkv_fwd(q, k, v, 4, o_part=o_part_s3)),
        ("split lse_part for 3 chunks", lambda: rf.splitkv_fwd(q, k, v, 4, lse_part=lse_part_s3)),
        ("merge out shape", lambda: rf.lse_merge(o_part_s3, lse_part_s3, out=torch.empty(1, 4, 8, 32, dtype=q.dtype, device=dev))),
        ("merge lse dtype", lambda: rf.lse_merge(o_part_s3, lse_part_s3, lse=torch.empty(1, 4, 8, dtype=torch.float64, device=dev))),
        ("bwd dk shape", lambda: rf.bwd(q, k, v, o, lse, dout, mask="causal", dk=torch.empty_like(q))),
        ("bwd dq dtype", lambda: rf.bwd(q, k, v, o, lse, dout, mask="causal", dq=torch.empty(q.shape, **f32))),
        ("bwd workspace small", lambda: rf.bwd(q, k, v, o, lse, dout, mask="causal", workspace=torch.empty(8, **f32))),
        ("rope out dtype", lambda: rf.rope_rotate(q, 10000.0, out=torch.empty(q.shape, **f32))),
        ("layernorm mean shape", lambda: rf.layernorm(x, gamma, beta, mean=torch.empty(5, **f32))),
        ("topk indices dtype", lambda: rf.softmax_topk(x, 4, indices=torch.empty(6, 4, dtype=torch.int64, device=dev))),
    ]


def test_wrong_output_buffers_are_refused():
    calls = _bad_buffer_calls()
    torch.cuda.synchronize()
    for what, call in calls:
        print(f"wrong buffer: {what}", flush=True)
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()
