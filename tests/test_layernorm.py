"""GPU parity of rf_layernorm_fwd with the float64 LayerNorm oracle.

Bound (derived from the arithmetic; the pages state no tolerance for this
path): y is rounded once to the output type, and before that is computed in
float32, where x - mean loses up to 2^-24 (|x| + |mean|) to cancellation.  So
every y element must lie within one unit in the last place of the output
type of the float64 reference (half an ulp of rounding, plus float32 error
that can move a value across a rounding midpoint) plus
4 * 2^-24 * ((|x| + |mean|) * rstd * |gamma| + |beta|); mean and rstd within
1e-5 relative (plus 1e-6 absolute for the mean).
"""
import numpy as np
import pytest
import torch

import attention_pass_cascaded_amd as rf
from oracle.layernorm import layer_norm
from workloads import LN_WORKLOAD, gen_layernorm

pytestmark = pytest.mark.gpu

MANT = {"f32": 23, "f16": 10, "bf16": 7}
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def ulp(ref, dt):
    a = np.maximum(np.abs(ref), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(a)) - MANT[dt])


def run(x, g, b, eps):
    dev = torch.device("cuda")
    xg, gg, bg = x.to(dev), g.to(dev), b.to(dev)
    y = torch.full_like(xg, float("nan"))
    mean = torch.full(x.shape[:-1], float("nan"), device=dev)
    rstd = torch.full(x.shape[:-1], float("nan"), device=dev)
    rf.layernorm(xg, gg, bg, eps, y=y, mean=mean, rstd=rstd)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy(), mean.cpu().double().numpy(), rstd.cpu().double().numpy()


def check(x, g, b, eps, dt, got):
    y, mean, rstd = got
    ry, rm, rr = layer_norm(x, g, b, eps)
    assert np.all(np.isfinite(y))
    err = np.abs(y - ry)
    xf = np.asarray(x.double() if hasattr(x, "double") else x, dtype=np.float64)
    gf = np.asarray(g.double() if hasattr(g, "double") else g, dtype=np.float64)
    bf = np.asarray(b.double() if hasattr(b, "double") else b, dtype=np.float64)
    arith = 4 * 2.0 ** -24 * ((np.abs(xf) + np.abs(rm)[:, None]) * rr[:, None] * np.abs(gf) + np.abs(bf))
    bound = ulp(ry, dt) + arith
    print(f"  y: max err/ulp {float((err / bound).max()) if err.size else 0:.3f}   "
          f"mean rel {float(np.abs(mean - rm).max() / max(1.0, np.abs(rm).max())) if rm.size else 0:.2e}")
    assert np.all(err <= bound), f"y off by more than one ulp: worst {float((err / bound).max()):.3f} ulp"
    np.testing.assert_allclose(mean, rm, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(rstd, rr, rtol=1e-5)


LN_CASES = [
    # dtype, rows, H
    ("bf16", 37, 4096),
    ("bf16", 3, 16384),
    ("f16", 64, 1000),
    ("f16", 5, 8),
    ("bf16", 11, 2056),
    ("f32", 100, 768),
    ("f32", 2, 8192),
    ("f32", 7, 4),
]


@pytest.mark.parametrize("dt,rows,H", LN_CASES)
def test_layernorm_matches_oracle(dt, rows, H):
    print(f"case layernorm {dt} rows={rows} H={H}", flush=True)
    x, g, b = gen_layernorm(rows, H, dt, seed=rows * 1000 + H)
    check(x, g, b, 1e-5, dt, run(x, g, b, 1e-5))


def test_layernorm_constant_rows_and_zero_rows():
    x = torch.full((4, 512), 3.25, dtype=torch.bfloat16)
    g = torch.ones(512, dtype=torch.bfloat16)
    b = torch.linspace(-1, 1, 512).to(torch.bfloat16)
    y, mean, rstd = run(x, g, b, 1e-5)
    assert np.all(mean == 3.25)
    np.testing.assert_array_equal(y, np.broadcast_to(b.float().numpy(), y.shape))
    empty = torch.empty((0, 512), dtype=torch.bfloat16)
    out = rf.layernorm(empty.cuda(), g.cuda(), b.cuda())
    assert out[0].shape == (0, 512)


def test_layernorm_unsupported_width():
    x = torch.zeros((2, 12), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(12, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rf.RFError):
        rf.layernorm(x, g, g)


def test_layernorm_full_size_workload_sampled():
    w = LN_WORKLOAD
    print(f"case layernorm full-size {w['name']}", flush=True)
    x, g, b = gen_layernorm(w["rows"], w["H"], w["dtype"], w["seed"], device="cuda")
    y, mean, rstd = rf.layernorm(x, g, b, w["eps"])
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(w["rows"], 64, replace=False)
    rows.sort()
    xs = x[rows].cpu()
    got = (y[rows].float().cpu().double().numpy(), mean[rows].cpu().double().numpy(), rstd[rows].cpu().double().numpy())
    check(xs, g.cpu(), b.cpu(), w["eps"], w["dtype"], got)
    assert torch.isfinite(y.float()).all()
