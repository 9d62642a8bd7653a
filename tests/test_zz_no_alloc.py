"""rf_attn_bwd_noalloc (row terms in the library's static per-GPU array)
against rf_attn_bwd (row terms in a caller workspace) through the C ABI: the
same kernels on the same inputs, so dq, dk and dv must agree bit for bit.
Two calls in a row on one GPU, the second smaller than the first, so the
second reads an array that still holds the first call's row terms; a third
call repeats the first shape after the smaller one."""
import pytest
import torch

import attention_pass_cascaded_amd as rf
from workloads import alibi_slopes, gen_grad_out, gen_qkv

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, mask, window, rope, alibi
    (2, 8, 4, 1000, 1000, 64, torch.float16, "causal", 0, 0.0, False),
    (1, 4, 2, 130, 257, 128, torch.bfloat16, "sliding", 96, 10000.0, True),
    (2, 8, 4, 1000, 1000, 64, torch.float16, "causal", 0, 0.0, False),
]


def run_case(B, Hq, Hkv, Nq, Nk, D, dtype, mask, window, rope, alibi, seed):
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in gen_qkv(B, Hq, Hkv, Nq, Nk, D, dtype, seed))
    do = gen_grad_out(q.shape, dtype, seed + 50).to(dev)
    slopes = torch.tensor(alibi_slopes(Hq), dtype=torch.float32, device=dev) if alibi else None
    kw = dict(scale=1.0 / D ** 0.5, mask=mask, window=window, rope_base=rope, alibi_slopes=slopes)
    o, lse = rf.fwd(q, k, v, **kw)
    ref = rf.bwd(q, k, v, o, lse, do, **kw)
    got = [torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))]
    rf.bwd_noalloc(q, k, v, o, lse, do, *got, **kw)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(g).all(), name
        assert torch.equal(g, r), f"{name}: max diff {(g.float() - r.float()).abs().max().item()}"


def test_noalloc_backward_matches_workspace_backward_on_consecutive_calls():
    for i, case in enumerate(CASES):
        print(f"noalloc case {i}: {case}", flush=True)
        run_case(*case, seed=70 + i)
