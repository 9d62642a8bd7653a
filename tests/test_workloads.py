"""Full-size parity: each workload at its real shape, launched exactly as
bench.py launches it, compared with the fp64 oracle on EVERY element of O and
LSE (the oracle runs one (batch, KV head) group at a time on the CPU), plus
properties every row must satisfy (finite O, finite LSE, |O| within the
largest |v| of its KV head).  The split-KV decode also has every partial
(o_c, lse_c) compared with the oracle's chunk.

For each workload the test prints, and appends as one JSON line to the file
named by the RF_PARITY_REPORT environment variable when it is set: the
largest |O - O64| and |LSE - LSE64|, the rounding floor max |rn(O64) - O64|
(what rounding the exact output once to the output dtype costs), the largest
distance of O from rn(O64) in spacings of the output grid, the element with
the largest O error, and the oracle's wall time.  The gate is the stated
max-abs tolerance (2e-3 fp16 and fp32, 1e-2 bf16) on O and LSE alike.
"""
import json
import os

import pytest
import torch

import attention_pass_cascaded_amd as rf
from oracle import report
from workloads import TABLE8_DECODE, WORKLOADS, gen_workload

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TOL = {"f32": 2e-3, "f16": 2e-3, "bf16": 1e-2}


def check_properties(w, k, v, o, lse):
    assert torch.isfinite(o).all()
    assert torch.isfinite(lse).all()  # every row of these workloads sees at least its own key
    vmax = v.float().abs().amax(dim=(2, 3))                     # [B, Hkv]
    vmax = vmax.repeat_interleave(w.Hq // w.Hkv, dim=1)         # [B, Hq]
    omax = o.float().abs().amax(dim=(2, 3))
    assert torch.all(omax <= vmax * (1 + 1e-2) + TOL[w.dtype])


def record(w, rep, extra=None):
    line = {"workload": w.name, "dtype": w.dtype, "tol": TOL[w.dtype],
            "elements_o": w.B * w.Hq * w.Nq * w.D, "rows": w.B * w.Hq * w.Nq, **rep, **(extra or {})}
    print(json.dumps(line), flush=True)
    path = os.environ.get("RF_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")


def gate(w, rep):
    tol = TOL[w.dtype]
    assert rep["max_abs_o"] <= tol, f"{w.name}: max|dO| {rep['max_abs_o']:.3e} > {tol} at {rep['worst']}"
    assert rep["max_abs_lse"] <= tol, f"{w.name}: max|dLSE| {rep['max_abs_lse']:.3e} > {tol}"


PREFILL = [w for w in WORKLOADS if not w.num_splits]
DECODE = [w for w in WORKLOADS if w.num_splits]


@pytest.mark.parametrize("w", PREFILL, ids=[w.name for w in PREFILL])
def test_prefill_workload_full_size(w):
    print(f"workload {w.name}", flush=True)
    q, k, v = gen_workload(w, device="cuda")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.Hq, w.Nq), float("nan"), device="cuda")
    rf.fwd(q, k, v, scale=w.scale, mask=w.mask, window=w.window, rope_base=w.rope_base, out=o, lse=lse)
    torch.cuda.synchronize()
    check_properties(w, k, v, o, lse)
    rep = report.compare_full(q, k, v, o, lse, w.scale, w.mask, w.window, w.rope_base, q.dtype)
    record(w, rep)
    gate(w, rep)


@pytest.mark.parametrize("w", DECODE, ids=[w.name for w in DECODE])
def test_decode_workload_full_size(w):
    print(f"workload {w.name}", flush=True)
    q, k, v = gen_workload(w, device="cuda")
    S = w.num_splits
    op = torch.full((w.B, w.Hq, w.Nq, S, w.D), float("nan"), device="cuda")
    lp = torch.full((w.B, w.Hq, w.Nq, S), float("nan"), device="cuda")
    rf.splitkv_fwd(q, k, v, S, scale=w.scale, mask=w.mask, window=w.window, rope_base=w.rope_base,
                   o_part=op, lse_part=lp)
    o, lse = rf.lse_merge(op, lp, out_dtype=q.dtype)
    torch.cuda.synchronize()
    assert torch.isfinite(op).all() and torch.isfinite(lp).all()
    check_properties(w, k, v, o, lse)
    rep = report.compare_full(q, k, v, o, lse, w.scale, w.mask, w.window, w.rope_base, q.dtype)
    pe_o, pe_l = report.compare_partials(q, k, v, op, lp, w.scale, S, w.mask, w.window, w.rope_base)
    record(w, rep, {"partials_max_abs_o": pe_o, "partials_max_abs_lse": pe_l})
    gate(w, rep)
    assert pe_o <= TOL[w.dtype] and pe_l <= TOL[w.dtype], (pe_o, pe_l)


@pytest.mark.parametrize("w", TABLE8_DECODE, ids=[w.name for w in TABLE8_DECODE])
def test_decode_geometry_full_size(w):
    """AttnFuse Table 8's decode geometries through rf.decode with the
    library's chunk-count rule (the launch bench.py times), every element
    against the oracle."""
    q, k, v = gen_workload(w, device="cuda")
    S = rf.num_splits_for(q, k)
    print(f"workload {w.name} num_splits={S}", flush=True)
    o, lse = rf.decode(q, k, v, num_splits=S, scale=w.scale)
    torch.cuda.synchronize()
    check_properties(w, k, v, o, lse)
    rep = report.compare_full(q, k, v, o, lse, w.scale, w.mask, w.window, w.rope_base, q.dtype)
    record(w, rep, {"num_splits": S})
    gate(w, rep)
