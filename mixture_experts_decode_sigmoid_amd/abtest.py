"""Paired A/B timing of builds of the library.

    python -m mixture_experts_decode_sigmoid_amd.abtest LIB_A LIB_B [LIB ...]
        --workloads v3_t1 v3_t8 [--rounds 24] [--batch 20]

Every build is loaded side by side in one process and gets its own layers
(and workspaces) on the same rotating weight copies.  Each round times one
batch of back-to-back calls per build between two HIP events on the launch
stream; the builds take turns, in reversed order every other round, so a slow
drift of the GPU (clock, memory state) reaches every build alike.  Printed per
workload: each build's median and mean microseconds per call, and the median
and quartiles of its per-round difference from the first build.  Two copies of
one build (an A/A run) show the method's resolution: about 0.3 us at one row.

This is the speed-test protocol of "sgl-amd-mono-upstream PR #27", Speed Tests
(each change timed against its parent, rounds in alternating order), with the
rounds interleaved within one process instead of across processes.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def run(paths, workloads, rounds=24, batch=20, copies=4, warmup=20):
    import torch
    sys.path.insert(0, ROOT)
    import fixtures
    import mixture_experts_decode_sigmoid_amd as moe
    names = [os.path.basename(p) for p in paths]
    libs = [moe.load_library(p, strict=False) for p in paths]
    results = {}
    for w in workloads:
        spec, case = fixtures.make_workload(w, device="cuda")
        keys = [k for k in case if k != "x"]
        cps = [case] + [{k: case[k].clone() for k in keys} for _ in range(copies - 1)]
        x = case["x"]
        T = x.shape[0]
        layers = []
        for L in libs:
            with moe.using(L):
                layers.append([moe.Layer(spec, dict(c, x=x), max_rows=T) for c in cps])
        out = torch.empty_like(x)
        stream = torch.cuda.current_stream()
        for L, ls in zip(libs, layers):
            with moe.using(L):
                for i in range(warmup):
                    ls[i % copies].forward(x, out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        us = [[] for _ in libs]
        for r in range(rounds):
            order = range(len(libs)) if r % 2 == 0 else reversed(range(len(libs)))
            for k in order:
                with moe.using(libs[k]):
                    a.record(stream)
                    for i in range(batch):
                        layers[k][i % copies].forward(x, out)
                    b.record(stream)
                    torch.cuda.synchronize()
                us[k].append(a.elapsed_time(b) * 1000.0 / batch)
        for k, L in enumerate(libs):
            with moe.using(L):
                if layers[k][0].read_error():
                    raise RuntimeError(f"{names[k]}: device error bits set on {w}")
        U = np.array(us)
        res = {}
        for k in range(len(libs)):
            d = U[k] - U[0]
            res[names[k]] = dict(median_us=round(float(np.median(U[k])), 2), mean_us=round(float(U[k].mean()), 2),
                                 diff_median=round(float(np.median(d)), 2),
                                 diff_q1=round(float(np.percentile(d, 25)), 2),
                                 diff_q3=round(float(np.percentile(d, 75)), 2))
        results[w] = res
        line = f"{w}: " + "  ".join(f"{n} {v['median_us']:.2f}" for n, v in res.items())
        line += "  | vs " + names[0] + ": " + "  ".join(
            f"{n} {v['diff_median']:+.2f} ({v['diff_q1']:+.2f}..{v['diff_q3']:+.2f})"
            for n, v in list(res.items())[1:])
        print(line, flush=True)
        del layers, cps, case
        torch.cuda.empty_cache()
    return results


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("libs", nargs="+", help="paths of the builds; the first is the reference")
    ap.add_argument("--workloads", nargs="+", required=True)
    ap.add_argument("--rounds", type=int, default=24)
    ap.add_argument("--batch", type=int, default=20)
    a = ap.parse_args()
    if len(a.libs) < 2:
        ap.error("give at least two builds")
    run(a.libs, a.workloads, a.rounds, a.batch)


if __name__ == "__main__":
    main()
