"""Parity at the largest KV head the boundary accepts (one head's K or V just
under 2 GiB: bf16, D = 128, Nk = 8,388,000), for the split-KV decode and the
fused forward.

With random data the output over millions of keys averages to ~0, which would
hide a wrong address.  So each query row gets "needle" keys: copies of 4·q at
fixed positions near the end of the head and near its middle.  Their scores
dominate, so O is the weighted mean of those far rows of V, and any 32-bit
offset overflow or misplaced tile would move it by O(1).  Reference: the fp64
oracle on all rows (K and V upcast once).  Tolerance: the bf16 bound 1e-2.
"""
import math

import numpy as np
import pytest
import torch

import attention_pass_cascaded_amd as rf
import oracle
from workloads import gen_qkv

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

NK = 8_388_000          # Nk * D * 2 bytes = 2,147,328,000 < 2^31
D = 128
HQ, HKV, NQ = 4, 1, 4
TOL = 1e-2


def needles(h, i):
    # key positions that row (h, i) is made to attend to: all visible under the
    # bottom-right causal alignment (query i sits at Nk - Nq + i)
    return [NK - NQ - 17 * h - 3 * i, NK - 2_000_003 + 101 * h + i, 6_000_000 + 977 * h + 13 * i]


@pytest.fixture(scope="module")
def problem():
    print(f"case max-size head: bf16 D={D} Nk={NK} Hq={HQ} Hkv={HKV} Nq={NQ}", flush=True)
    q, k, v = gen_qkv(1, HQ, HKV, NQ, NK, D, "bf16", seed=11, device="cuda")
    k.mul_(0.1)
    for h in range(HQ):
        for i in range(NQ):
            for j in needles(h, i):
                k[0, 0, j] = (4.0 * q[0, h, i].float()).to(k.dtype)
    torch.cuda.synchronize()
    k64 = k.float().cpu().double().numpy()
    v64 = v.float().cpu().double().numpy()
    q64 = q.float().cpu().double().numpy()
    return q, k, v, q64, k64, v64


def compare(o, lse, ro, rl, what):
    got_o = o.float().cpu().double().numpy()
    got_l = lse.cpu().double().numpy()
    err_o = float(np.abs(got_o - ro).max())
    err_l = float(np.abs(got_l - rl).max())
    print(f"{what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} max|O|={float(np.abs(ro).max()):.3f}", flush=True)
    assert np.abs(ro).max() > 0.1  # the needles dominate: O is not ~0
    assert err_o <= TOL and err_l <= TOL


def test_decode_at_largest_kv_head(problem):
    q, k, v, q64, k64, v64 = problem
    scale = 1 / math.sqrt(D)
    o, lse = rf.decode(q, k, v, num_splits=64, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q64, k64, v64, scale)
    compare(o, lse, ro, rl, "decode")


def test_fused_forward_causal_at_largest_kv_head(problem):
    q, k, v, q64, k64, v64 = problem
    scale = 1 / math.sqrt(D)
    o, lse = rf.fwd(q, k, v, scale=scale, mask="causal")
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q64, k64, v64, scale, mask="causal")
    compare(o, lse, ro, rl, "fused forward, causal")


# D = 64: the largest head is twice as long (Nk * 64 * 2 bytes just under
# 2 GiB).  The 16-bit D = 64 forward also runs as key halves (layouts 1 and 2),
# whose second group starts half-way through the keys; with one query block
# and no mask the halves are [0, ~8.4M) and [~8.4M, Nk), and the needles sit
# in both, so the on-chip merge of the two halves is checked at the largest
# offsets the boundary accepts.
NK64 = 16_777_000       # Nk * 64 * 2 bytes = 2,147,456,000 < 2^31


def needles64(h, i):
    return [NK64 - 1 - 29 * h - 5 * i, 8_400_001 + 131 * h + 7 * i, 3_000_000 + 977 * h + 13 * i]


@pytest.fixture(scope="module")
def problem64():
    print(f"case max-size head: bf16 D=64 Nk={NK64} Hq={HQ} Hkv={HKV} Nq={NQ}", flush=True)
    q, k, v = gen_qkv(1, HQ, HKV, NQ, NK64, 64, "bf16", seed=12, device="cuda")
    k.mul_(0.1)
    for h in range(HQ):
        for i in range(NQ):
            for j in needles64(h, i):
                k[0, 0, j] = (4.0 * q[0, h, i].float()).to(k.dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q.float().cpu().double().numpy(), k.float().cpu().double().numpy(),
                              v.float().cpu().double().numpy(), 1 / 8)
    return q, k, v, ro, rl


@pytest.mark.parametrize("layout", ["0", "1", "2"])
def test_fused_forward_d64_layouts_at_largest_kv_head(problem64, monkeypatch, layout):
    q, k, v, ro, rl = problem64
    monkeypatch.setenv("RF_ATTN_KEY_HALVES", layout)
    print(f"case max-size D=64 forward, layout {layout}", flush=True)
    o, lse = rf.fwd(q, k, v, scale=1 / 8)
    torch.cuda.synchronize()
    compare(o, lse, ro, rl, f"fused forward D=64, layout {layout}")
