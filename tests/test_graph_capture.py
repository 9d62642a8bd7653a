"""The entry points under HIP graph capture.

The library allocates nothing and clears nothing with memset, and launches
only on the caller's stream, so a caller can capture a whole step (forward,
split-KV decode and merge, backward, LayerNorm, softmax -> TopK) into one
graph and replay it.  Each replay here runs on fresh inputs written into the
captured buffers, with eager work and synchronisations between replays, and
must reproduce the eager results of the same calls bit for bit (every kernel
is deterministic).
"""
import math

import pytest
import torch

import attention_pass_cascaded_amd as rf
from workloads import gen_grad_out, gen_layernorm, gen_logits, gen_qkv

pytestmark = pytest.mark.gpu


def test_captured_step_matches_eager_on_every_replay():
    print("case graph capture: fwd + decode + merge + bwd + layernorm + topk", flush=True)
    dev = "cuda"
    q, k, v = gen_qkv(1, 4, 2, 300, 300, 64, "f16", seed=21, device=dev)
    do = gen_grad_out(q.shape, "f16", seed=22, device=dev)
    qd, kd, vd = gen_qkv(2, 8, 2, 1, 2048, 128, "bf16", seed=23, device=dev)
    x, gam, bet = gen_layernorm(64, 1024, "bf16", seed=24, device=dev)
    logits = gen_logits(128, 256, "bf16", seed=25, device=dev)
    # an unmasked grid of one 128-row block per CU (8 heads x 32 blocks): the
    # 8-wave key-halves layout on a 256-CU GPU
    q2, k2, v2 = gen_qkv(1, 8, 8, 4096, 4096, 64, "f16", seed=26, device=dev)

    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(1 * 4 * 300, device=dev)
    S = 16
    op = torch.empty((2, 8, 1, S, 128), device=dev)
    lp = torch.empty((2, 8, 1, S), device=dev)
    od = torch.empty_like(qd)
    lsed = torch.empty(qd.shape[:3], device=dev)
    y = torch.empty_like(x)
    mean = torch.empty(x.shape[:1], device=dev)
    rstd = torch.empty(x.shape[:1], device=dev)
    vals = torch.empty((128, 8), device=dev)
    idx = torch.empty((128, 8), dtype=torch.int32, device=dev)
    o2 = torch.empty_like(q2)
    lse2 = torch.empty(q2.shape[:3], device=dev)
    outs = (o, lse, dq, dk, dv, od, lsed, y, mean, rstd, vals, idx, o2, lse2)

    def step():
        rf.fwd(q, k, v, scale=0.125, mask="causal", rope_base=10000.0, out=o, lse=lse)
        rf.bwd(q, k, v, o, lse, do, scale=0.125, mask="causal", rope_base=10000.0, dq=dq, dk=dk, dv=dv,
               workspace=ws)
        rf.splitkv_fwd(qd, kd, vd, S, scale=1 / math.sqrt(128), o_part=op, lse_part=lp)
        rf.lse_merge(op, lp, out=od, lse=lsed)
        rf.layernorm(x, gam, bet, 1e-5, y=y, mean=mean, rstd=rstd)
        rf.softmax_topk(logits, 8, values=vals, indices=idx)
        rf.fwd(q2, k2, v2, scale=0.125, out=o2, lse=lse2)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    inputs = (q, k, v, do, qd, kd, vd, x, logits, q2, k2, v2)
    for rep in range(3):
        gen = torch.Generator(device=dev).manual_seed(100 + rep)
        for t in inputs:
            t.copy_(torch.randn(t.shape, generator=gen, device=dev, dtype=torch.float32).to(t.dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replayed = [t.clone() for t in outs]
        for t in outs:
            t.zero_()
        step()  # eager, same inputs
        torch.cuda.synchronize()
        names = ("o", "lse", "dq", "dk", "dv", "o_dec", "lse_dec", "y", "mean", "rstd", "vals", "idx",
                 "o_halves", "lse_halves")
        assert len(names) == len(outs)
        for name, a, b in zip(names, replayed, outs):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from eager"
