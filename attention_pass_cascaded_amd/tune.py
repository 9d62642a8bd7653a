"""Offline tile/occupancy sweep for the compile-time knobs of the kernels.

For every setting of a knob group the library is built in-tree under
``_build/tune/`` (``build.build(extra_flags=-D..., out=...)``), each build is
timed in a child process of its own (``RF_ATTN_LIB`` names it) on the
workloads that group affects, and the fastest setting of each group is
written to ``csrc/tuned.hpp`` with ``--write`` (the kernels take their
defaults from that header; ``-D`` still overrides it).  Rebuild afterwards
(``python -m attention_pass_cascaded_amd.build``).

Needs a GPU.  Usage:

    python -m attention_pass_cascaded_amd.tune [--write] [--steps 100] [--warmup 20]
    python -m attention_pass_cascaded_amd.tune --from-log sweep.log   # header from a printed sweep

Groups (the knobs only change instances that the named workloads run):
  fwd  RF_FWD_WAVES_D64 in {2, 3, 4}: waves per SIMD of the 16-bit D = 64
       forward without RoPE or ALiBi (register budget 512 / waves);
       timed on the causal fp16 B4 H12 N4096 D64 forward and the same shape
       unmasked.
  bwd  RF_BWD_DQ_WAVES in {2, 3} x RF_BWD_KV_WAVES in {2, 3} x RF_BWD_BQ64 in
       {32, 64}: waves per SIMD of the D = 64 dq and dk/dv kernels and the
       dk/dv kernel's query tile; timed on the backward of the causal fp16
       B4 H12 N4096 D64 workload.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import itertools
import json
import os
import subprocess
import sys

from . import build as B

ROOT = B.ROOT
TUNE_DIR = os.path.join(B.OBJ, "tune")
HEADER = os.path.join(B.CSRC, "tuned.hpp")

GROUPS = {
    "fwd": {"knobs": {"RF_FWD_WAVES_D64": [2, 3, 4]},
            "runs": [("prefill", "causal_f16_b4h12_n4096_d64", "causal"), ("prefill", "causal_f16_b4h12_n4096_d64", "none")]},
    "bwd": {"knobs": {"RF_BWD_DQ_WAVES": [2, 3], "RF_BWD_KV_WAVES": [2, 3], "RF_BWD_BQ64": [32, 64]},
            "runs": [("backward", "causal_f16_b4h12_n4096_d64", "causal")]},
}

# Child process: time one library build on the given runs; prints one JSON line.
_TIMER = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import dataclasses, torch
import attention_pass_cascaded_amd as rf
from workloads import by_name, gen_workload, gen_grad_out
steps, warmup = int(sys.argv[2]), int(sys.argv[3])
out = {}
for kind, name, mask in json.loads(sys.argv[4]):
    w = dataclasses.replace(by_name(name), mask=mask)
    q, k, v = gen_workload(w, device="cuda")
    o, lse = rf.fwd(q, k, v, scale=w.scale, mask=w.mask)
    if kind == "prefill":
        call = lambda: rf.fwd(q, k, v, scale=w.scale, mask=w.mask, out=o, lse=lse)
    else:
        do = gen_grad_out(q.shape, w.dtype, w.seed + 100, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(w.B * w.Hq * w.Nq, dtype=torch.float32, device="cuda")
        call = lambda: rf.bwd(q, k, v, o, lse, do, scale=w.scale, mask=w.mask, dq=dq, dk=dk, dv=dv, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    out[f"{kind}:{name}:{mask}"] = a.elapsed_time(b) / steps
print(json.dumps(out), flush=True)
"""


def settings(group):
    knobs = GROUPS[group]["knobs"]
    names = list(knobs)
    for vals in itertools.product(*(knobs[n] for n in names)):
        yield dict(zip(names, vals))


def tag(group, setting):
    return group + "_" + "_".join(f"{k.split('_', 2)[-1].lower()}{v}" for k, v in setting.items())


def build_one(group, setting):
    lib = os.path.join(TUNE_DIR, tag(group, setting), "librfattn.so")
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    B.build(extra_flags=[f"-D{k}={v}" for k, v in setting.items()], out=lib)
    return lib


def time_lib(lib, runs, steps, warmup):
    env = dict(os.environ, RF_ATTN_LIB=lib)
    r = subprocess.run([sys.executable, "-c", _TIMER, ROOT, str(steps), str(warmup), json.dumps(runs)],
                       env=env, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"timing {lib} failed:\n{r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def write_header(winners, table, path=HEADER):
    lines = ["// Compile-time tile and occupancy knobs of the kernels: the fastest setting",
             "// of each group in the sweep of attention_pass_cascaded_amd/tune.py on one",
             "// MI355X (ms per call; every setting that was built and timed is listed).",
             "// A -D on the compiler line overrides a value here.",
             "#pragma once", ""]
    for group, rows in table.items():
        lines.append(f"// {group}:")
        for setting, res, total in rows:
            s = ", ".join(f"{k}={v}" for k, v in setting.items())
            t = ", ".join(f"{k.split(':')[0]} {k.split(':')[2]} {v:.4f}" for k, v in res.items())
            lines.append(f"//   {s}: {t}")
        lines.append("")
    for group in GROUPS:
        for k, v in winners[group].items():
            lines += [f"#ifndef {k}", f"#define {k} {v}", "#endif"]
    open(path, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description="tile/occupancy sweep; writes csrc/tuned.hpp with --write")
    ap.add_argument("--write", action="store_true")
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--groups", default=",".join(GROUPS))
    ap.add_argument("--from-log", default=None, metavar="FILE",
                    help="write the header from the JSON lines a previous sweep printed (no build, no GPU)")
    args = ap.parse_args()
    if args.from_log:
        winners = header_from_log(args.from_log)
        print(json.dumps({"winners": winners}), f"wrote {HEADER}", flush=True)
        return
    groups = [g for g in args.groups.split(",") if g]
    jobs = [(g, s) for g in groups for s in settings(g)]
    print(f"building {len(jobs)} libraries under {TUNE_DIR}", flush=True)
    libs = [None] * len(jobs)
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {ex.submit(build_one, *j): i for i, j in enumerate(jobs)}
        for f in cf.as_completed(futs):
            libs[futs[f]] = f.result()
            print(f"built {libs[futs[f]]}", flush=True)
    table = {g: [] for g in groups}
    for (g, s), lib in zip(jobs, libs):
        res = time_lib(lib, GROUPS[g]["runs"], args.steps, args.warmup)
        total = sum(res.values())
        table[g].append((s, res, total))
        print(json.dumps({"group": g, "setting": s, "ms": res, "total_ms": total}), flush=True)
    winners = {g: min(rows, key=lambda r: r[2])[0] for g, rows in table.items()}
    print(json.dumps({"winners": winners}), flush=True)
    if args.write:
        for g in GROUPS:
            if g not in winners:  # a group not swept keeps its current values
                winners[g] = {k: current_value(k) for k in GROUPS[g]["knobs"]}
        write_header(winners, table)
        print(f"wrote {HEADER}", flush=True)


def header_from_log(log, path=HEADER):
    """Write the header from the JSON lines a sweep printed; returns the winners."""
    table = {}
    for line in open(log):
        if line.startswith('{"group"'):
            d = json.loads(line)
            table.setdefault(d["group"], []).append((d["setting"], d["ms"], d["total_ms"]))
    winners = {g: min(rows, key=lambda r: r[2])[0] for g, rows in table.items()}
    for g in GROUPS:
        if g not in winners:  # a group not swept keeps its current values
            winners[g] = {k: current_value(k, path) for k in GROUPS[g]["knobs"]}
    write_header(winners, table, path)
    return winners


def current_value(knob, path=HEADER):
    for line in open(path):
        if line.startswith(f"#define {knob} "):
            return int(line.split()[2])
    raise KeyError(knob)


if __name__ == "__main__":
    main()
