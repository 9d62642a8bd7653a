"""The causal forward's work-group order covers every (head, query block) once.

Causal grids are dealt heaviest query blocks first; when the whole grid is
resident at launch, every other run of (number of CUs) groups is taken in
reverse so that each CU gets a mix of heavy and light blocks.  The order is a
permutation of the blocks: here O and LSE start as NaN and every element
must be written, for grids below, at and above the snake's threshold (the
number of CUs times the groups resident per CU), and sampled rows must match
the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import attention_pass_cascaded_amd as rf
import oracle
from workloads import gen_qkv

pytestmark = pytest.mark.gpu

# (B, H, N, D, dtype, rope_base): 16 query blocks per head
CASES = [
    (1, 17, 2048, 64, "f16", 0.0),        # 272 groups: one full run and a partial one
    (1, 33, 2048, 64, "f16", 0.0),        # 528 groups: the second run reversed, a partial third
    (4, 12, 2048, 64, "f16", 10000.0),    # 768 groups: three full runs (RoPE, all resident)
    (4, 12, 4096, 64, "f16", 0.0),        # 1536 groups: more than are resident, plain order
    (2, 16, 2048, 128, "bf16", 0.0),      # D = 128 instance
]


@pytest.mark.parametrize("B,H,N,D,dtype,rope_base", CASES)
def test_every_block_written_once(B, H, N, D, dtype, rope_base):
    print(f"case grid order: B={B} H={H} N={N} D={D} {dtype} rope={rope_base}", flush=True)
    q, k, v = gen_qkv(B, H, H, N, N, D, dtype, seed=31, device="cuda")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    scale = 1.0 / np.sqrt(D)
    rf.fwd(q, k, v, scale=scale, mask="causal", rope_base=rope_base, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    # rows of the last and first query blocks of a few heads against the oracle
    rng = np.random.default_rng(5)
    heads = [(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))]
    rows = [(b, h, i) for b, h in heads for i in (0, 127, 128, N // 2, N - 129, N - 1)]
    q64 = q.float().cpu().double().numpy()
    k64 = k.float().cpu().double().numpy()
    v64 = v.float().cpu().double().numpy()
    ro, rl = oracle.attention_rows(q64, k64, v64, scale, rows, "causal", 0, rope_base)
    idx = tuple(np.array(rows).T)
    got_o = o.float().cpu().double().numpy()[idx]
    got_l = lse.cpu().double().numpy()[idx]
    tol = 2e-3 if dtype == "f16" else 1e-2
    assert float(np.abs(got_o - ro).max()) <= tol
    assert float(np.abs(got_l - rl).max()) <= tol
