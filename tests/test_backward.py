"""GPU parity of the backward (rf_attn_bwd through the C ABI) with the fp64
chain-rule oracle (oracle/backward.py).

The GPU path takes o and lse from the GPU forward (as a training step does);
the oracle differentiates the exact forward.  The method states tolerances
for forward outputs only, so the gradient bound is derived from the
arithmetic: every product rounds P or dS once to the input type (unit
roundoff u = 2^-11 for fp16, 2^-8 for bf16), D_i uses the rounded o, and each
gradient is rounded once on output.  The error of each element is a few u
times the size of the terms summed into it, so the test bounds the largest
error of each tensor by C_u * u * max|reference| + 2^-16 with C_u = 8 (fp16)
and C_u = 4 (bf16), checked on every element (the 2^-16 floor covers float32
summation-order residue where the exact gradient is 0).  Outputs are poisoned with NaN
before the call so an unwritten element fails.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import attention_pass_cascaded_amd as rf
from oracle.backward import attention_backward
from workloads import alibi_slopes, by_name, gen_grad_out, gen_qkv

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
C_U = {"f16": 8.0, "bf16": 4.0}
DT = {"f16": torch.float16, "bf16": torch.bfloat16}
# absolute floor: dP_ij - D_i is a difference of two float32 dot products
# summed in different orders; where the exact difference is 0 (a row that
# sees one key) the kernel keeps a float32 rounding residue of this size
FLOOR = 2.0 ** -16


def run(q, k, v, do, scale, mask, window, rope, slopes):
    dev = torch.device("cuda")
    qg, kg, vg, dog = (t.to(dev) for t in (q, k, v, do))
    o, lse = rf.fwd(qg, kg, vg, scale=scale, mask=mask, window=window, rope_base=rope, alibi_slopes=slopes)
    dq = torch.full_like(qg, float("nan"))
    dk = torch.full_like(kg, float("nan"))
    dv = torch.full_like(vg, float("nan"))
    rf.bwd(qg, kg, vg, o, lse, dog, scale=scale, mask=mask, window=window, rope_base=rope,
           alibi_slopes=slopes, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(name, got, ref, dt):
    got = got.detach().float().cpu().double().numpy()
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{name}: non-finite element"
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    bound = C_U[dt] * U[dt] * scale + FLOOR
    print(f"  {name}: max err {err:.3e}  max|ref| {scale:.3e}  err/(u*max|ref|) {err / (U[dt] * max(scale, 1e-30)):.2f}")
    assert err <= bound, f"{name}: max err {err:.3e} > {bound:.3e}"


BWD_CASES = [
    # dtype, D, B, Hq, Hkv, Nq, Nk, mask, window, rope, alibi
    ("f16", 64, 1, 2, 2, 200, 200, "none", 0, 0.0, False),
    ("f16", 64, 2, 4, 2, 300, 300, "causal", 0, 0.0, False),
    ("bf16", 64, 1, 2, 1, 130, 260, "causal", 0, 0.0, False),
    ("f16", 64, 1, 2, 1, 100, 60, "causal", 0, 0.0, False),
    ("f16", 128, 1, 2, 2, 257, 257, "sliding", 50, 0.0, False),
    ("bf16", 128, 1, 4, 1, 190, 190, "causal", 0, 10000.0, False),
    ("f16", 64, 1, 2, 2, 200, 200, "causal", 0, 10000.0, False),
    ("bf16", 64, 1, 2, 2, 333, 333, "sliding", 37, 500.0, False),
    ("f16", 64, 1, 2, 2, 150, 150, "causal", 0, 0.0, True),
    ("bf16", 128, 1, 4, 2, 140, 140, "causal", 0, 10000.0, True),
    ("f16", 64, 1, 1, 1, 1, 1, "none", 0, 0.0, False),
    ("bf16", 128, 1, 2, 2, 5, 300, "none", 0, 0.0, False),
    ("f16", 128, 1, 2, 2, 64, 64, "sliding", 1, 0.0, False),
]


@pytest.mark.parametrize("dt,D,B,Hq,Hkv,Nq,Nk,mask,window,rope,alibi", BWD_CASES)
def test_bwd_matches_oracle(dt, D, B, Hq, Hkv, Nq, Nk, mask, window, rope, alibi):
    seed = zlib.crc32(repr(("bwd", dt, D, B, Hq, Hkv, Nq, Nk, mask, window, rope, alibi)).encode()) % 10_000
    q, k, v = gen_qkv(B, Hq, Hkv, Nq, Nk, D, dt, seed)
    do = gen_grad_out((B, Hq, Nq, D), dt, seed + 1)
    scale = 1.0 / math.sqrt(D)
    slopes = alibi_slopes(Hq) if alibi else None
    print(f"case bwd {dt} D={D} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} {mask} W={window} rope={rope} alibi={alibi}", flush=True)
    dq, dk, dv = run(q, k, v, do, scale, mask, window, rope, slopes)
    rq, rk, rv = attention_backward(q, k, v, do, scale, mask, window, rope, slopes)
    check("dq", dq, rq, dt)
    check("dk", dk, rk, dt)
    check("dv", dv, rv, dt)


def test_bwd_keys_nobody_sees_get_zero():
    # Nq > Nk with a causal mask: every key is seen by some row; with a
    # window of 1 and Nq < Nk the leading keys are seen by no query.
    q, k, v = gen_qkv(1, 2, 2, 40, 200, 64, "f16", 7)
    do = gen_grad_out((1, 2, 40, 64), "f16", 8)
    dq, dk, dv = run(q, k, v, do, 0.125, "sliding", 1, 0.0, None)
    unseen = 200 - 40
    assert torch.all(dk[:, :, :unseen].float() == 0) and torch.all(dv[:, :, :unseen].float() == 0)


def test_bwd_is_deterministic():
    q, k, v = gen_qkv(1, 4, 2, 300, 300, 64, "bf16", 9)
    do = gen_grad_out((1, 4, 300, 64), "bf16", 10)
    a = run(q, k, v, do, 0.125, "causal", 0, 10000.0, None)
    b = run(q, k, v, do, 0.125, "causal", 0, 10000.0, None)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_full_size_causal_workload_one_head():
    """The causal fp16 B=4 H=12 N=4096 D=64 workload at full size, as timed;
    one head (b=1, h=7) checked element by element (MHA: dk, dv of KV head 7
    come from query head 7 only)."""
    w = by_name("causal_f16_b4h12_n4096_d64")
    q, k, v = gen_qkv(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, w.dtype, w.seed)
    do = gen_grad_out(q.shape, w.dtype, w.seed + 100)
    print("case bwd full-size causal_f16_b4h12_n4096_d64 head (1, 7)", flush=True)
    dq, dk, dv = run(q, k, v, do, w.scale, w.mask, w.window, w.rope_base, None)
    rq, rk, rv = attention_backward(q[1:2, 7:8], k[1:2, 7:8], v[1:2, 7:8], do[1:2, 7:8], w.scale, w.mask,
                                    w.window, w.rope_base)
    check("dq", dq[1:2, 7:8], rq, "f16")
    check("dk", dk[1:2, 7:8], rk, "f16")
    check("dv", dv[1:2, 7:8], rv, "f16")
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
