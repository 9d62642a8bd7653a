#!/usr/bin/env python3
"""Benchmark of the fused cascaded-reduction attention on one MI355X.

A step is one fused forward (rf_attn_fwd) over the causal fp16 prefill
workload B=4 H=12 N=4096 D=64 (the workload the AttnFuse listing's Tables 1-3
time on H100 NVL), inputs resident in HBM.  The split-KV decode (GQA 32q/8kv,
D=128, 32768 cached keys, 64 chunks of 512; AttnFuse Table 8 geometry) and the
other prefill variants are timed in the same run and reported as secondary
objects.  Prints ONE JSON line.

Work counted (algorithmic, not what the kernels happen to execute):
  flops = 4 * D per visible (query, key) pair (Q.K^T and P.V, 2 each);
  bytes = q, k, v read once + o written once (+ lse, float32).
Timing: torch.cuda.Event on the stream the kernels are launched on (the
current stream).  Each workload first runs untimed for 0.3 s so the GPU clock
reaches its loaded steady state, then W untimed warmup steps, then K timed
steps back to back.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused attn-fwd TFLOP/s (prefill) + decode HBM GB/s, % of MI355X roofline"
HEADLINE = "causal_f16_b4h12_n4096_d64"
DECODE = "gqa_decode_bf16_b16_32q8kv_nk32768_d128"
VARIANTS = ["rope_causal_f16_b4h12_n2048_d64", "sliding256_bf16_b8h16_n8192_d128"]

# MI355X published peaks: 256 CUs at 2.4 GHz.
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}  # dense MFMA
PEAK_HBM_GBS = 8000.0
PAGES_HEADLINE_MS = 0.488  # AttnFuse, causal fp16 B4 H12 N4096 D64, H100 NVL (Table 3)

# Files whose content defines each kernel: HBM counter figures are used only
# while these are unchanged since the counters were taken.
KERNEL_SOURCES = {
    "fwd": ["attention_pass_cascaded_amd/csrc/fwd_kernel.hpp", "attention_pass_cascaded_amd/csrc/common.hpp"],
    "decode": ["attention_pass_cascaded_amd/csrc/decode_mfma_kernel.hpp", "attention_pass_cascaded_amd/csrc/common.hpp"],
    "layernorm": ["attention_pass_cascaded_amd/csrc/layernorm_kernel.hpp", "attention_pass_cascaded_amd/csrc/common.hpp"],
}


def kernel_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def visible_pairs(Nq: int, Nk: int, mask: str, window: int = 0) -> int:
    """(query, key) pairs a head computes: query i at position Nk - Nq + i."""
    total = 0
    for i in range(Nq):
        p = Nk - Nq + i
        if mask == "none":
            total += Nk
        else:
            hi = min(p, Nk - 1)
            lo = 0 if mask == "causal" else max(0, p - window + 1)
            total += max(0, hi - lo + 1)
    return total


def alg_flops(w) -> float:
    return 4.0 * w.D * visible_pairs(w.Nq, w.Nk, w.mask, w.window) * w.B * w.Hq


def alg_bytes(w) -> float:
    es = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    qo = 2 * w.B * w.Hq * w.Nq * w.D * es
    kv = 2 * w.B * w.Hkv * w.Nk * w.D * es
    return float(qo + kv + 4 * w.B * w.Hq * w.Nq)


def traffic_from_profiles(kind: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if still valid."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    hsh = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not hsh or hsh.group(1) != kernel_hash(kind):
        return None
    return float(m.group(1))


CLOCK_WARM_S = 0.3  # untimed run-in before the warmup steps: lets the GPU clock settle


def time_loop(fn, steps: int, warmup: int) -> float:
    """ms per call: a clock run-in, `warmup` untimed calls, then `steps` timed calls."""
    import torch
    t_end = time.perf_counter() + CLOCK_WARM_S
    while time.perf_counter() < t_end:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def run_prefill(w, steps, warmup):
    import torch
    import attention_pass_cascaded_amd as rf
    from workloads import gen_workload
    q, k, v = gen_workload(w, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")

    def step():
        rf.fwd(q, k, v, scale=w.scale, mask=w.mask, window=w.window, rope_base=w.rope_base, out=o, lse=lse)

    ms = time_loop(step, steps, warmup)
    flops = alg_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    byts = alg_bytes(w)
    gbs = byts / (ms * 1e-3) / 1e9
    traffic = traffic_from_profiles("fwd", w.name)
    res = {
        "workload": w.name, "ms": ms, "TFLOP/s": tflops, "GB/s": gbs,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": tflops / peak, "traffic": traffic},
        "hbm_frac": gbs / PEAK_HBM_GBS,
        "alg_gflop": flops / 1e9, "alg_mb": byts / 1e6,
    }
    return res, (q, k, v)


def run_backward(w, steps, warmup):
    """rf_attn_bwd (row terms + dk/dv + dq kernels) on a prefill workload, with
    o and lse from the fused forward.  Algorithmic flops: 5 products of 2*D
    flops per visible pair (S recomputed, dP, dV, dK, dQ) = 2.5x the forward;
    the kernels execute 7 (S and dP are recomputed in both the dk/dv and the
    dq kernel), reported as executed_TFLOP/s."""
    import torch
    import attention_pass_cascaded_amd as rf
    from workloads import gen_grad_out, gen_workload
    q, k, v = gen_workload(w, device="cuda")
    do = gen_grad_out(q.shape, w.dtype, w.seed + 100, device="cuda")
    o, lse = rf.fwd(q, k, v, scale=w.scale, mask=w.mask, window=w.window, rope_base=w.rope_base)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(w.B * w.Hq * w.Nq, dtype=torch.float32, device="cuda")

    def step():
        rf.bwd(q, k, v, o, lse, do, scale=w.scale, mask=w.mask, window=w.window, rope_base=w.rope_base,
               dq=dq, dk=dk, dv=dv, workspace=ws)

    ms = time_loop(step, steps, warmup)
    flops = 2.5 * alg_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    return {"workload": w.name, "ms": ms, "TFLOP/s": tflops, "executed_TFLOP/s": tflops * 7.0 / 5.0,
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                         "frac": tflops / peak, "traffic": None},
            "alg_gflop": flops / 1e9}


def run_layernorm(steps, warmup):
    """rf_layernorm_fwd on the LayerNorm workload: HBM-bound (x read once, y
    written once; gamma, beta, mean and rstd are counted too)."""
    import torch
    import attention_pass_cascaded_amd as rf
    from workloads import LN_WORKLOAD as w, gen_layernorm
    x, g, b = gen_layernorm(w["rows"], w["H"], w["dtype"], w["seed"], device="cuda")
    y = torch.empty_like(x)
    mean = torch.empty(w["rows"], dtype=torch.float32, device="cuda")
    rstd = torch.empty_like(mean)

    def step():
        rf.layernorm(x, g, b, w["eps"], y=y, mean=mean, rstd=rstd)

    ms = time_loop(step, steps, warmup)
    es = x.element_size()
    byts = 2 * w["rows"] * w["H"] * es + 2 * w["H"] * es + 8 * w["rows"]
    gbs = byts / (ms * 1e-3) / 1e9
    return {"workload": w["name"], "ms": ms, "GB/s": gbs,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": traffic_from_profiles("layernorm", w["name"])},
            "alg_mb": byts / 1e6}


def run_topk(steps, warmup):
    """rf_softmax_topk on the router workload (logits read once; values and
    indices written)."""
    import torch
    import attention_pass_cascaded_amd as rf
    from workloads import TOPK_WORKLOAD as w, gen_logits
    x = gen_logits(w["rows"], w["E"], w["dtype"], w["seed"], device="cuda")
    vals = torch.empty((w["rows"], w["k"]), dtype=torch.float32, device="cuda")
    idx = torch.empty((w["rows"], w["k"]), dtype=torch.int32, device="cuda")
    ms = time_loop(lambda: rf.softmax_topk(x, w["k"], values=vals, indices=idx), steps, warmup)
    byts = x.numel() * x.element_size() + 8 * w["rows"] * w["k"]
    gbs = byts / (ms * 1e-3) / 1e9
    return {"workload": w["name"], "ms": ms, "GB/s": gbs,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": None},
            "alg_mb": byts / 1e6}


def run_decode(w, steps, warmup):
    import torch
    import attention_pass_cascaded_amd as rf
    from workloads import gen_workload
    q, k, v = gen_workload(w, device="cuda")
    S = w.num_splits
    op = torch.empty((w.B, w.Hq, w.Nq, S, w.D), dtype=torch.float32, device="cuda")
    lp = torch.empty((w.B, w.Hq, w.Nq, S), dtype=torch.float32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")

    def part():
        rf.splitkv_fwd(q, k, v, S, scale=w.scale, mask=w.mask, window=w.window, rope_base=w.rope_base,
                       o_part=op, lse_part=lp)

    def merge():
        rf.lse_merge(op, lp, out_dtype=q.dtype, out=o, lse=lse)

    def step():
        part()
        merge()

    ms = time_loop(step, steps, warmup)
    ms_part = time_loop(part, steps, warmup)
    ms_merge = time_loop(merge, steps, warmup)
    byts = alg_bytes(w)
    gbs = byts / (ms * 1e-3) / 1e9
    gbs_part = byts / (ms_part * 1e-3) / 1e9
    traffic = traffic_from_profiles("decode", w.name)
    return {
        "workload": w.name, "value": gbs, "unit": "GB/s", "ms_per_step": ms,
        "ms_partial_kernel": ms_part, "ms_merge_kernel": ms_merge,
        "roofline": {"bound": "hbm", "achieved": gbs_part, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs_part / PEAK_HBM_GBS, "traffic": traffic},
        "step_frac_of_hbm_peak": gbs / PEAK_HBM_GBS,
        "alg_mb": byts / 1e6, "alg_gflop": alg_flops(w) / 1e9,
    }


def cpu_baseline(w, q, k, v, heads: int):
    """The fp64 oracle on the workload (or batch 0's first `heads` heads)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    if heads <= 0:
        qs, ks, vs = q.cpu(), k.cpu(), v.cpu()
        heads = w.B * w.Hq
    else:
        qs = q[:1, :heads].cpu()
        ks = k[:1, : max(1, heads * w.Hkv // w.Hq)].cpu()
        vs = v[:1, : max(1, heads * w.Hkv // w.Hq)].cpu()
    t0 = time.perf_counter()
    if threadpool_limits is not None:
        with threadpool_limits(limits=cores):
            oracle.attention(qs, ks, vs, w.scale, w.mask, w.window, w.rope_base)
    else:
        oracle.attention(qs, ks, vs, w.scale, w.mask, w.window, w.rope_base)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.D * visible_pairs(w.Nq, w.Nk, w.mask, w.window) * heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"whole {w.name} workload" if heads == w.B * w.Hq else
                       f"batch 0, heads 0..{heads - 1} of {w.name} ({heads}/{w.B * w.Hq} of the workload)")
                      + f", {flops / 1e9:.2f} GFLOP in {dt:.1f} s, float64 numpy three-pass oracle"}


def rotation_sweep(steps: int, warmup: int, Ns=(512, 1024, 2048, 4096, 8192, 16384)):
    """Fused RoPE vs rotate-first, causal fp16 B=4 H=12 D=64 (AttnFuse Table 4's comparison).

    speedup = (rotate q + rotate k + attention without RoPE) / (attention with fused RoPE);
    above 1 the fused kernel wins.  N* is interpolated where the speedup crosses 1.
    """
    import torch
    import attention_pass_cascaded_amd as rf
    from workloads import gen_qkv
    rows = []
    for N in Ns:
        q, k, v = gen_qkv(4, 12, 12, N, N, 64, "f16", seed=3, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((4, 12, N), dtype=torch.float32, device="cuda")
        qr, kr = torch.empty_like(q), torch.empty_like(k)

        def fused():
            rf.fwd(q, k, v, scale=0.125, mask="causal", rope_base=10000.0, out=o, lse=lse)

        def rotate_first():
            rf.rope_rotate(q, 10000.0, 0, out=qr)
            rf.rope_rotate(k, 10000.0, 0, out=kr)
            rf.fwd(qr, kr, v, scale=0.125, mask="causal", out=o, lse=lse)

        def plain():
            rf.fwd(q, k, v, scale=0.125, mask="causal", out=o, lse=lse)

        def rot_only():
            rf.rope_rotate(q, 10000.0, 0, out=qr)
            rf.rope_rotate(k, 10000.0, 0, out=kr)

        t = {name: time_loop(fn, steps, warmup) for name, fn in
             (("fused_ms", fused), ("rotate_first_ms", rotate_first), ("plain_causal_ms", plain),
              ("rotate_qk_ms", rot_only))}
        t["speedup_fused_over_rotate_first"] = t["rotate_first_ms"] / t["fused_ms"]
        t["N"] = N
        rows.append(t)
        print(json.dumps(t), flush=True)
    nstar = None
    for a, b in zip(rows, rows[1:]):
        sa, sb = a["speedup_fused_over_rotate_first"], b["speedup_fused_over_rotate_first"]
        if (sa - 1) * (sb - 1) < 0:
            la, lb = math.log(a["N"]), math.log(b["N"])
            nstar = math.exp(la + (1 - sa) * (lb - la) / (sb - sa))
    print(json.dumps({"rotation_calculus_crossover_N": nstar,
                      "fused_wins_at": [r["N"] for r in rows if r["speedup_fused_over_rotate_first"] > 1]}))


def copy_calibration(nbytes: int, steps: int):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4, "launches": steps}))


def copy_rate(nbytes: int = 1 << 30, steps: int = 20) -> float:
    """GB/s (read + write) of a plain device copy: the HBM rate a streaming
    kernel can practically reach on this machine, reported next to the 8 TB/s peak."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    ms = time_loop(lambda: dst.copy_(src), steps, 3)
    return 2 * nbytes / (ms * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--only", default=None, help="time a single workload (for profiling runs)")
    ap.add_argument("--only-bwd", default=None, metavar="WORKLOAD", help="time the backward of one prefill workload")
    ap.add_argument("--only-layernorm", action="store_true", help="time the LayerNorm workload only")
    ap.add_argument("--only-topk", action="store_true", help="time the softmax-TopK workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads of batch 0 for the oracle (0: whole workload)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--rotation-sweep", action="store_true",
                    help="fused RoPE vs rotate-first over N (prints one JSON line per N)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported. Prefill shards "
              "over (batch, head) and decode over (batch, KV head) with no exchange, so each GPU runs "
              "this one-GPU workload on its share.", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import by_name
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    if args.rotation_sweep:
        rotation_sweep(args.steps, args.warmup)
        return

    if args.only_topk:
        print(json.dumps(run_topk(args.steps, args.warmup)), flush=True)
        return
    if args.only_layernorm:
        print(json.dumps(run_layernorm(args.steps, args.warmup)), flush=True)
        return
    if args.only_bwd:
        print(json.dumps(run_backward(by_name(args.only_bwd), args.steps, args.warmup)), flush=True)
        return
    if args.only:
        w = by_name(args.only)
        res = run_decode(w, args.steps, args.warmup) if w.num_splits else run_prefill(w, args.steps, args.warmup)[0]
        print(json.dumps(res), flush=True)
        return

    w = by_name(HEADLINE)
    head, (q, k, v) = run_prefill(w, args.steps, args.warmup)
    print(f"# headline {w.name}: {head['ms']:.4f} ms, {head['TFLOP/s']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    dec = run_decode(by_name(DECODE), args.steps, args.warmup)
    print(f"# decode: {dec['ms_per_step']:.4f} ms, {dec['value']:.0f} GB/s", file=sys.stderr, flush=True)
    variants = {}
    for name in VARIANTS:
        r, _ = run_prefill(by_name(name), args.steps, args.warmup)
        variants[name] = {"ms": r["ms"], "TFLOP/s": r["TFLOP/s"], "GB/s": r["GB/s"],
                          "mfma_frac": r["roofline"]["frac"], "hbm_frac": r["hbm_frac"]}
        print(f"# {name}: {r['ms']:.4f} ms", file=sys.stderr, flush=True)
    bwd = run_backward(w, max(1, args.steps // 4), max(1, args.warmup // 4))
    print(f"# backward {w.name}: {bwd['ms']:.4f} ms, {bwd['TFLOP/s']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    ln = run_layernorm(args.steps, args.warmup)
    print(f"# layernorm {ln['workload']}: {ln['ms']:.4f} ms, {ln['GB/s']:.0f} GB/s", file=sys.stderr, flush=True)
    tk = run_topk(args.steps, args.warmup)
    print(f"# softmax-topk {tk['workload']}: {tk['ms']:.4f} ms, {tk['GB/s']:.0f} GB/s", file=sys.stderr, flush=True)
    copy_gbs = copy_rate()
    print(f"# device copy: {copy_gbs:.0f} GB/s", file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, q, k, v, args.cpu_heads)

    # The pages' own time for this exact workload (AttnFuse's dispatched
    # kernel, Table 3 / Table 2 BN=64 winner: 0.488 ms on an H100 NVL),
    # turned into TFLOP/s with the same algorithmic flop count.  Another
    # machine's figure: context for the ratio, not a target.
    pages_tflops = alg_flops(w) / (PAGES_HEADLINE_MS * 1e-3) / 1e12
    line = {
        "metric": METRIC, "value": head["TFLOP/s"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": head["TFLOP/s"] / pages_tflops,
        "baseline_ref": {"value": pages_tflops, "unit": "TFLOP/s", "ms": PAGES_HEADLINE_MS,
                         "hardware": "H100 NVL", "source": "AttnFuse Table 3 (dispatched kernel)"},
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1), GPU generator)",
        "config": {"workload": w.name, "B": w.B, "H": w.Hq, "N": w.Nq, "D": w.D, "mask": w.mask,
                   "global_batch": w.B, "seq_len": w.Nq, "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "decode": dec,
        "variants": variants,
        "backward": bwd,
        "layernorm": ln,
        "softmax_topk": tk,
        "hbm_copy_GB/s": copy_gbs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
