"""GPU parity of rf_softmax_topk with the float64 softmax -> TopK oracle.

Indices are compared bit-exactly: both sides select on the exact input
values with ties to the lower index, so the result is unique (bf16 logits
make ties common).  Values: the pages state no tolerance for this path; the
kernel forms p = 2^((x - m) log2 e) / l in float32, so each value may be off
by a few 2^-24 relative per step: the bound used is
2^-24 * (E + 8 + |x - m| log2 e) relative, checked element by element.
"""
import numpy as np
import pytest
import torch

import attention_pass_cascaded_amd as rf
from oracle.topk import softmax_topk
from workloads import TOPK_WORKLOAD, gen_logits

pytestmark = pytest.mark.gpu


def check(x, k, vals, idx):
    rv, ri = softmax_topk(x, k)
    idx = idx.cpu().numpy()
    vals = vals.cpu().double().numpy()
    np.testing.assert_array_equal(idx, ri)
    xf = np.asarray(x.double() if hasattr(x, "double") else x, dtype=np.float64)
    E = xf.shape[1]
    gap = (xf.max(axis=1)[:, None] - np.take_along_axis(xf, ri, 1)) * 1.4426950408889634
    tol = 2.0 ** -24 * (E + 8 + gap)
    rel = np.abs(vals - rv) / rv
    print(f"  max rel err {float(rel.max()):.2e} (bound >= {float(tol.min()):.2e})")
    assert np.all(rel <= tol)


CASES = [
    # dtype, rows, E, k   (16-lane groups for E <= 256 and k <= 16, else whole
    # wavefronts; 16-bit rows take the packed-key kernel, f32 the pair kernel)
    ("bf16", 33, 256, 8),
    ("bf16", 7, 1024, 64),
    ("f16", 50, 100, 5),
    ("f16", 9, 7, 3),
    ("bf16", 17, 200, 12),
    ("f16", 40, 256, 16),
    ("f32", 9, 64, 64),
    ("f32", 5, 1, 1),
    ("bf16", 3, 777, 13),
]


@pytest.mark.parametrize("dt,rows,E,k", CASES)
def test_softmax_topk_matches_oracle(dt, rows, E, k):
    print(f"case topk {dt} rows={rows} E={E} k={k}", flush=True)
    x = gen_logits(rows, E, dt, seed=rows * 100 + E)
    vals, idx = rf.softmax_topk(x.cuda(), k)
    torch.cuda.synchronize()
    check(x, k, vals, idx)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_softmax_topk_unaligned_rows(dt):
    """Rows that start 2 bytes past a 16-byte boundary (E a multiple of 8):
    the element loads fall back from 16-byte chunks to single elements."""
    rows, E, k = 21, 256, 8
    flat = gen_logits(1, rows * E + 1, dt, seed=4242).reshape(-1)
    print(f"case topk unaligned {dt}", flush=True)
    xg = flat.cuda()[1:].view(rows, E)
    assert xg.data_ptr() % 16 == 2
    vals, idx = rf.softmax_topk(xg, k)
    torch.cuda.synchronize()
    check(flat[1:].view(rows, E), k, vals, idx)


def test_softmax_topk_all_ties():
    x = torch.zeros((4, 96), dtype=torch.bfloat16)
    vals, idx = rf.softmax_topk(x.cuda(), 10)
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), torch.arange(10, dtype=torch.int32).repeat(4, 1))
    assert torch.allclose(vals.cpu(), torch.full((4, 10), 1.0 / 96), rtol=1e-6)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("k", [4, 12])
def test_softmax_topk_signed_zeros_and_neg_inf(dt, k):
    # -0 and +0 are equal values (ties go to the lower index); -inf entries
    # are valid and get p = 0
    row = [-0.0, 0.0, -0.0, 1.0, float("-inf"), -0.5, 0.0, -0.0, float("-inf"), -3.0] * 5
    x = torch.tensor([row, row[::-1]], dtype=getattr(torch, {"bf16": "bfloat16", "f16": "float16"}[dt]))
    vals, idx = rf.softmax_topk(x.cuda(), k)
    torch.cuda.synchronize()
    check(x, k, vals, idx)
    # the five 1.0 entries first, then the zeros of either sign by index
    expect = [3, 13, 23, 33, 43, 0, 1, 2, 6, 7, 10, 11][:k]
    assert idx[0].tolist() == expect


def test_softmax_topk_rejects_bad_k():
    x = torch.zeros((2, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(rf.RFError):
        rf.softmax_topk(x, 17)


def test_softmax_topk_full_size_workload_sampled():
    w = TOPK_WORKLOAD
    print(f"case topk full-size {w['name']}", flush=True)
    x = gen_logits(w["rows"], w["E"], w["dtype"], w["seed"], device="cuda")
    vals, idx = rf.softmax_topk(x, w["k"])
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(w["rows"], 256, replace=False))
    check(x[rows].cpu(), w["k"], vals[rows].cpu(), idx[rows].cpu())
    assert torch.all((idx >= 0) & (idx < w["E"]))
