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
    "fwd": ["attention_pass_cascaded_amd/csrc/fwd_kernel.hpp", "attention_pass_cascaded_amd/csrc/common.hpp",
            "attention_pass_cascaded_amd/csrc/tuned.hpp"],
    "decode": ["attention_pass_cascaded_amd/csrc/decode_mfma_kernel.hpp", "attention_pass_cascaded_amd/csrc/common.hpp"],
    "layernorm": ["attention_pass_cascaded_amd/csrc/layernorm_kernel.hpp", "attention_pass_cascaded_amd/csrc/common.hpp"],
    "bwd": ["attention_pass_cascaded_amd/csrc/bwd_kernel.hpp", "attention_pass_cascaded_amd/csrc/fwd_kernel.hpp",
            "attention_pass_cascaded_amd/csrc/common.hpp", "attention_pass_cascaded_amd/csrc/tuned.hpp"],
    "topk": ["attention_pass_cascaded_amd/csrc/topk_kernel.hpp", "attention_pass_cascaded_amd/csrc/common.hpp"],
    "merge": ["attention_pass_cascaded_amd/csrc/merge_kernel.hpp", "attention_pass_cascaded_amd/csrc/common.hpp"],
    "rope": ["attention_pass_cascaded_amd/csrc/rope_kernel.hpp", "attention_pass_cascaded_amd/csrc/common.hpp"],
}
GRAPH_TIMING = True  # bench.py --no-graph turns the captured-graph timings off (counter passes)


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


def time_steps(fn, steps: int, warmup: int) -> dict:
    """Per-call times in ms: a clock run-in, `warmup` untimed calls, then
    `steps` calls back to back with an event recorded between consecutive
    calls on the current stream.  Returns mean (total / steps), median, min."""
    import torch
    t_end = time.perf_counter() + CLOCK_WARM_S
    while time.perf_counter() < t_end:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    mid = steps // 2
    median = per[mid] if steps % 2 else 0.5 * (per[mid - 1] + per[mid])
    return {"mean": ev[0].elapsed_time(ev[steps]) / steps, "median": median, "min": per[0]}


def time_loop(fn, steps: int, warmup: int) -> float:
    """Mean ms per call (see time_steps)."""
    return time_steps(fn, steps, warmup)["mean"]


def time_graph(fn, calls: int = 20, replays: int = 50) -> float:
    """Mean ms per call of `fn` replayed from a captured HIP graph holding
    `calls` back-to-back calls: the GPU time of a short launch sequence
    without the host's per-call cost (Python, ctypes, launch), the way a
    serving loop issues decode steps.  The calls must not allocate."""
    import torch
    if not GRAPH_TIMING:
        return float("nan")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (replays * calls)


def run_prefill(w, steps, warmup, alibi=False):
    import torch
    import attention_pass_cascaded_amd as rf
    from workloads import alibi_slopes, gen_workload
    q, k, v = gen_workload(w, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
    slopes = torch.tensor(alibi_slopes(w.Hq), dtype=torch.float32, device="cuda") if alibi else None

    def step():
        rf.fwd(q, k, v, scale=w.scale, mask=w.mask, window=w.window, rope_base=w.rope_base, out=o, lse=lse,
               alibi_slopes=slopes)

    t = time_steps(step, steps, warmup)
    ms = t["mean"]
    flops = alg_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    byts = alg_bytes(w)
    gbs = byts / (ms * 1e-3) / 1e9
    traffic = traffic_from_profiles("fwd", w.name)
    res = {
        "workload": w.name, "ms": ms, "ms_median": t["median"], "ms_min": t["min"],
        "TFLOP/s": tflops, "GB/s": gbs,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": tflops / peak, "traffic": traffic},
        "hbm_frac": gbs / PEAK_HBM_GBS,
        "alg_gflop": flops / 1e9, "alg_mb": byts / 1e6,
    }
    return res, (q, k, v, o, lse)


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
    call = lambda: rf.softmax_topk(x, w["k"], values=vals, indices=idx)
    ms = time_loop(call, steps, warmup)
    # a few-microsecond kernel: eager calls are bound by the host's per-call
    # cost, so the roofline uses the time inside a captured graph
    ms_graph = time_graph(call)
    byts = x.numel() * x.element_size() + 8 * w["rows"] * w["k"]
    gbs = byts / ((ms if ms_graph != ms_graph else ms_graph) * 1e-3) / 1e9  # eager time without the graph
    return {"workload": w["name"], "ms": ms, "ms_graph": ms_graph if ms_graph == ms_graph else None, "GB/s": gbs,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": None},
            "alg_mb": byts / 1e6}


def run_decode(w, steps, warmup, num_splits=None, keep=False):
    """Split-KV partials + merge on a decode workload.  num_splits defaults to
    the workload's own (the decode config fixes 64 chunks of 512); the
    decode geometries take the library's rule (rf_splitkv_num_splits)."""
    import torch
    import attention_pass_cascaded_amd as rf
    from workloads import gen_workload
    q, k, v = gen_workload(w, device="cuda")
    S = int(num_splits or w.num_splits or rf.num_splits_for(q, k))
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

    t = time_steps(step, steps, warmup)
    ms = t["mean"]
    ms_part = time_loop(part, steps, warmup)
    ms_merge = time_loop(merge, steps, warmup)
    ms_graph = time_graph(step, calls=10, replays=max(5, min(50, steps // 4)))
    byts = alg_bytes(w)
    gbs = byts / (ms * 1e-3) / 1e9
    gbs_part = byts / (ms_part * 1e-3) / 1e9
    traffic = traffic_from_profiles("decode", w.name)
    res = {
        "workload": w.name, "num_splits": S, "value": gbs, "unit": "GB/s", "ms_per_step": ms,
        "ms_median": t["median"], "ms_min": t["min"], "ms_step_graph": ms_graph if ms_graph == ms_graph else None,
        "GB/s_step_graph": byts / (ms_graph * 1e-3) / 1e9 if ms_graph == ms_graph else None,
        "ms_partial_kernel": ms_part, "ms_merge_kernel": ms_merge,
        "roofline": {"bound": "hbm", "achieved": gbs_part, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs_part / PEAK_HBM_GBS, "traffic": traffic},
        "step_frac_of_hbm_peak": gbs / PEAK_HBM_GBS,
        "alg_mb": byts / 1e6, "alg_gflop": alg_flops(w) / 1e9,
    }
    if keep:
        return res, (q, k, v, o, lse)
    return res


def decode_geometries(steps, warmup, sweep=False):
    """AttnFuse Table 8's three decode geometries at batch 1 and 16 (bf16,
    Q.N = 1), each with num_splits from the library's rule; with ``sweep``
    also every power of two from 8 to 256 chunks."""
    from workloads import TABLE8_DECODE
    out = []
    for w in TABLE8_DECODE:
        r = run_decode(w, steps, warmup)
        row = {"workload": w.name, "num_splits": r["num_splits"], "ms_per_step": r["ms_per_step"],
               "ms_median": r["ms_median"], "GB/s": r["value"], "step_frac_of_hbm_peak": r["step_frac_of_hbm_peak"],
               "ms_step_graph": r["ms_step_graph"], "GB/s_step_graph": r["GB/s_step_graph"],
               "partial_GB/s": r["roofline"]["achieved"], "partial_frac": r["roofline"]["frac"]}
        if sweep:
            row["sweep_ms"] = {}
            for S in (8, 16, 32, 64, 128, 256):
                if S <= w.Nk:
                    row["sweep_ms"][S] = run_decode(w, steps, warmup, num_splits=S)["ms_per_step"]
        print(f"# decode {w.name}: S={row['num_splits']} {row['ms_per_step']:.4f} ms {row['GB/s']:.0f} GB/s",
              file=sys.stderr, flush=True)
        out.append(row)
    return out


VARIANT_SET = [  # AttnFuse Tables 6-7's variants, at the causal headline's shape
    ("dense", dict(mask="none")),
    ("causal", dict(mask="causal")),
    ("sliding_w256", dict(mask="sliding", window=256)),
    ("causal_alibi", dict(mask="causal", alibi=True)),
    ("dense_rope", dict(mask="none", rope_base=10000.0)),
    ("sliding_w256_rope", dict(mask="sliding", window=256, rope_base=10000.0)),
]


def variants_table(steps, warmup):
    """Time each variant at B=4 H=12 N=4096 D=64 fp16 (absolute time and
    roofline fraction; flops over the variant's own visible pairs)."""
    import dataclasses
    from workloads import by_name
    base = by_name(HEADLINE)
    rows = {}
    for name, kw in VARIANT_SET:
        kw = dict(kw)
        alibi = kw.pop("alibi", False)
        w = dataclasses.replace(base, name=f"{name}_f16_b4h12_n4096_d64", mask=kw.get("mask", "none"),
                                window=kw.get("window", 0), rope_base=kw.get("rope_base", 0.0))
        r, _ = run_prefill(w, steps, warmup, alibi=alibi)
        rows[name] = {"ms": r["ms"], "ms_median": r["ms_median"], "TFLOP/s": r["TFLOP/s"],
                      "mfma_frac": r["roofline"]["frac"], "GB/s": r["GB/s"], "hbm_frac": r["hbm_frac"],
                      "alg_gflop": r["alg_gflop"]}
        print(f"# variant {name}: {r['ms']:.4f} ms {r['TFLOP/s']:.0f} TFLOP/s", file=sys.stderr, flush=True)
    return rows


def host_cores() -> tuple[int, dict]:
    """Threads for the oracle: the cores this process may run on
    (sched_getaffinity), capped by the cgroup CPU quota when one is set."""
    aff = len(os.sched_getaffinity(0))
    quota = None
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = max(1, math.ceil(int(q) / int(per)))
    except (OSError, ValueError):
        pass
    return (min(aff, quota) if quota else aff), {"affinity_cores": aff, "cgroup_quota_cores": quota}


def blas_backend() -> str:
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{d.get('internal_api')} {d.get('version')} ({d.get('threading_layer')}, {d.get('architecture')})"
                for d in threadpool_info() if d.get("user_api") == "blas"]
        if libs:
            return "; ".join(libs)
    except Exception:  # pragma: no cover
        pass
    import numpy
    return str(numpy.__config__.CONFIG.get("Build Dependencies", {}).get("blas", {}).get("name"))


def oracle_leg(runs):
    """The fp64 oracle beside each config (every element of every config),
    on the host cores: its wall time (slice copies excluded) and the kernel's
    whole-output error against it.  ``runs``: list of (workload, (q, k, v, o, lse))."""
    from oracle import report
    from threadpoolctl import threadpool_limits
    cores, core_info = host_cores()
    per_config, parity = [], []
    with threadpool_limits(limits=cores):
        for w, (q, k, v, o, lse) in runs:
            t0 = time.perf_counter()
            rep = report.compare_full(q, k, v, o, lse, w.scale, w.mask, w.window, w.rope_base, q.dtype)
            wall = time.perf_counter() - t0
            flops = alg_flops(w)
            tol = {"f32": 2e-3, "f16": 2e-3, "bf16": 1e-2}[w.dtype]
            per_config.append({"workload": w.name, "oracle_s": rep["oracle_s"], "wall_s_with_compare": wall,
                               "TFLOP/s": flops / rep["oracle_s"] / 1e12, "sample": "whole workload"})
            parity.append({"workload": w.name, "tol": tol, "max_abs_o": rep["max_abs_o"],
                           "max_abs_lse": rep["max_abs_lse"], "floor": rep["floor"], "ulps": rep["ulps"],
                           "worst": rep["worst"],
                           "pass": rep["max_abs_o"] <= tol and rep["max_abs_lse"] <= tol})
            print(f"# oracle {w.name}: {rep['oracle_s']:.1f} s; max|dO| {rep['max_abs_o']:.2e} "
                  f"(floor {rep['floor']:.2e}, {rep['ulps']:.0f} ulp) max|dLSE| {rep['max_abs_lse']:.2e}",
                  file=sys.stderr, flush=True)
    return cores, core_info, per_config, parity


def sample_clock(fn, seconds: float = 1.5):
    """Shader clock while ``fn`` runs back to back: rocm-smi (or amd-smi) is
    started as a child process while another thread keeps the GPU busy.
    Returns the MHz values it printed for the graphics clock, or the reason
    none was read."""
    import subprocess
    import threading
    import torch
    stop = threading.Event()

    def load():
        while not stop.is_set():
            for _ in range(10):
                fn()
            torch.cuda.synchronize()

    th = threading.Thread(target=load, daemon=True)
    th.start()
    time.sleep(min(0.5, seconds / 3))
    found, raw = [], ""
    try:
        for cmd in (["rocm-smi", "--showclocks", "--json"], ["amd-smi", "metric", "--clock", "--json"]):
            try:
                r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
            except (OSError, subprocess.TimeoutExpired) as e:
                raw += f"{cmd[0]}: {e}; "
                continue
            raw += r.stdout[-400:]
            for key, val in re.findall(r'"([^"]*(?:sclk|gfx|GFX)[^"]*)"\s*:\s*"?([^",}]*)', r.stdout):
                found += [int(x) for x in re.findall(r"(\d{3,4})\s*[Mm][Hh]z", val)]
            if found:
                return {"tool": cmd[0], "MHz": sorted(set(found))}
    finally:
        stop.set()
        th.join()
    return {"tool": None, "MHz": None, "raw": raw[-600:]}


def shape_sweep(steps: int, warmup: int):
    """The fused forward across shapes: B=4, H=16, N = Nq = Nk from 1024 to
    16384, D 64 and 128, fp16 and bf16, causal and unmasked; one JSON line per
    shape (time, TFLOP/s, fraction of the MFMA peak).  The number of timed
    calls shrinks for the large shapes so every shape takes about 0.2 s."""
    import dataclasses
    from workloads import Workload
    for D in (64, 128):
        for dt in ("f16", "bf16"):
            for mask in ("causal", "none"):
                for N in (1024, 2048, 4096, 8192, 16384):
                    w = Workload(f"{mask}_{dt}_b4h16_n{N}_d{D}", B=4, Hq=16, Hkv=16, Nq=N, Nk=N, D=D, dtype=dt,
                                 scale=1.0 / math.sqrt(D), mask=mask, seed=42)
                    est_ms = alg_flops(w) / (800e12 * 1e-3)  # at ~800 TFLOP/s
                    n = int(max(10, min(steps, 200.0 / max(est_ms, 1e-3))))
                    r, _ = run_prefill(dataclasses.replace(w), n, max(3, min(warmup, n // 4)))
                    print(json.dumps({"shape": w.name, "B": w.B, "H": w.Hq, "N": N, "D": D, "dtype": dt, "mask": mask,
                                      "ms": r["ms"], "ms_median": r["ms_median"], "TFLOP/s": r["TFLOP/s"],
                                      "mfma_frac": r["roofline"]["frac"], "steps": n}), flush=True)


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
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (timing and parity)")
    ap.add_argument("--decode-sweep", action="store_true",
                    help="decode geometries with every chunk count 8..256 (prints one JSON line)")
    ap.add_argument("--variants", action="store_true", help="the variant table only (prints one JSON line)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="the fused forward over N, D, dtype and mask at B=4 H=16 (one JSON line per shape)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the captured-graph timings of the short launches (for counter passes)")
    ap.add_argument("--rotation-sweep", action="store_true",
                    help="fused RoPE vs rotate-first over N (prints one JSON line per N)")
    args = ap.parse_args()
    global GRAPH_TIMING
    GRAPH_TIMING = not args.no_graph

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported. Prefill shards "
              "over (batch, head) and decode over (batch, KV head) with no exchange, so each GPU runs "
              "this one-GPU workload on its share.", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import WORKLOADS, by_name
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    if args.rotation_sweep:
        rotation_sweep(args.steps, args.warmup)
        return
    if args.shape_sweep:
        shape_sweep(args.steps, args.warmup)
        return
    if args.decode_sweep:
        print(json.dumps({"decode_geometries": decode_geometries(args.steps, args.warmup, sweep=True)}), flush=True)
        return
    if args.variants:
        print(json.dumps({"variants_table": variants_table(args.steps, args.warmup)}), flush=True)
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
        res = (run_decode(w, args.steps, args.warmup) if w.num_splits or w.Nq == 1
               else run_prefill(w, args.steps, args.warmup)[0])
        print(json.dumps(res), flush=True)
        return

    # the headline: one step = one fused forward over the causal fp16 workload
    w = by_name(HEADLINE)
    head, head_t = run_prefill(w, args.steps, args.warmup)
    print(f"# headline {w.name}: {head['ms']:.4f} ms (median {head['ms_median']:.4f}, min {head['ms_min']:.4f}), "
          f"{head['TFLOP/s']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    import attention_pass_cascaded_amd as rf
    q, k, v, o, lse = head_t
    clock = sample_clock(lambda: rf.fwd(q, k, v, scale=w.scale, mask=w.mask, out=o, lse=lse))
    print(f"# shader clock under the headline's load: {clock}", file=sys.stderr, flush=True)

    # every config in the same run: timing, then the oracle beside it
    configs, runs = {}, []
    for cw in WORKLOADS:
        if cw.name == HEADLINE:
            r, t = head, head_t
        elif cw.num_splits:
            r, t = run_decode(cw, args.steps, args.warmup, keep=True)
        else:
            r, t = run_prefill(cw, args.steps, args.warmup)
        runs.append((cw, t))
        if cw.num_splits:
            configs[cw.name] = {"ms": r["ms_per_step"], "ms_median": r["ms_median"], "ms_min": r["ms_min"],
                                "GB/s": r["value"], "num_splits": r["num_splits"],
                                "ms_partial_kernel": r["ms_partial_kernel"], "ms_merge_kernel": r["ms_merge_kernel"],
                                "roofline": r["roofline"], "step_frac_of_hbm_peak": r["step_frac_of_hbm_peak"]}
        else:
            configs[cw.name] = {"ms": r["ms"], "ms_median": r["ms_median"], "ms_min": r["ms_min"],
                                "TFLOP/s": r["TFLOP/s"], "GB/s": r["GB/s"], "roofline": r["roofline"],
                                "hbm_frac": r["hbm_frac"]}
        print(f"# {cw.name}: {configs[cw.name]['ms']:.4f} ms", file=sys.stderr, flush=True)
    dec = configs[DECODE]
    geo = decode_geometries(args.steps, args.warmup)
    var = variants_table(args.steps, args.warmup)
    bwd = run_backward(w, max(1, args.steps // 4), max(1, args.warmup // 4))
    print(f"# backward {w.name}: {bwd['ms']:.4f} ms, {bwd['TFLOP/s']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    ln = run_layernorm(args.steps, args.warmup)
    print(f"# layernorm {ln['workload']}: {ln['ms']:.4f} ms, {ln['GB/s']:.0f} GB/s", file=sys.stderr, flush=True)
    tk = run_topk(args.steps, args.warmup)
    print(f"# softmax-topk {tk['workload']}: {tk['ms']:.4f} ms, {tk['GB/s']:.0f} GB/s", file=sys.stderr, flush=True)
    copy_gbs = copy_rate()
    print(f"# device copy: {copy_gbs:.0f} GB/s", file=sys.stderr, flush=True)

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        cores, core_info, per_config, parity = oracle_leg(runs)
        for pc in per_config:
            configs[pc["workload"]]["oracle_s"] = pc["oracle_s"]
        for pr in parity:
            configs[pr["workload"]]["max_abs_o"] = pr["max_abs_o"]
            configs[pr["workload"]]["max_abs_lse"] = pr["max_abs_lse"]
        hp = next(pc for pc in per_config if pc["workload"] == HEADLINE)
        cpu = {"value": hp["TFLOP/s"], "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": f"whole {HEADLINE} workload ({alg_flops(w) / 1e9:.2f} GFLOP) in {hp['oracle_s']:.1f} s, "
                         "float64 numpy three-pass oracle, one (batch, KV head) group at a time",
               "blas": blas_backend(), **core_info, "per_config": per_config}

    # The pages' own time for this exact workload (AttnFuse's dispatched
    # kernel, Table 3 / Table 2 BN=64 winner: 0.488 ms on an H100 NVL),
    # turned into TFLOP/s with the same algorithmic flop count.  Another
    # machine's figure: context for the ratio, not a target.
    pages_tflops = alg_flops(w) / (PAGES_HEADLINE_MS * 1e-3) / 1e12
    line = {
        "metric": METRIC, "value": head["TFLOP/s"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms"],
        "ms_per_step_median": head["ms_median"], "ms_per_step_min": head["ms_min"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": head["TFLOP/s"] / pages_tflops,
        "baseline_ref": {"value": pages_tflops, "unit": "TFLOP/s", "ms": PAGES_HEADLINE_MS,
                         "hardware": "H100 NVL", "source": "AttnFuse Table 3 (dispatched kernel)"},
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1), GPU generator)",
        "config": {"workload": w.name, "B": w.B, "H": w.Hq, "N": w.Nq, "D": w.D, "mask": w.mask,
                   "global_batch": w.B, "seq_len": w.Nq, "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "shader_clock": clock,
        "configs": configs,
        "parity": parity,
        "decode": dec,
        "decode_geometries": geo,
        "variants_table": var,
        "backward": bwd,
        "layernorm": ln,
        "softmax_topk": tk,
        "hbm_copy_GB/s": copy_gbs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
