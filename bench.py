"""Benchmark of the fused decode MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

Headline workload: the DeepSeek-V3-shaped layer (hidden 7168, expert
intermediate 2048, 256 routed experts top-8 in 8 groups keep 4, one shared
expert, FP8 E4M3 weights with 128x128 fp32 block scales) at 1 decode row.
A step is one fused layer call (one kernel launch) on one row of seeded
synthetic input.  Four full copies of the weights (router included) rotate
between steps so that a repeat cannot be served from the 256 MB last-level
cache; inputs are resident in HBM before timing starts.

value = achieved HBM GB/s on the algorithmic bytes (every used expert's
weights and scales once, plus the router weights), B_alg / mean call time.
The same figures at 8 rows (2 requests x 4 MTP rows) and 64 independent rows
are reported under "extra".  cpu_baseline times the fp64 oracle on the
host's cores on the one-row layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
N_COPIES = 4
HEADLINE = "v3_t1"
EXTRA = ("v3_t8", "v3_t64")
# one GPU's share of the layer under 8-way tensor parallelism (own weights)
EXTRA_SHARD = ("v3tp8_t1", "v3tp8_t8")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("moe_kernels.hip", "moe_kernels_res.hip", "moe_api.cpp", "moe_internal.h"):
        with open(os.path.join(ROOT, "mixture_experts_decode_sigmoid_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary of this
    workload, if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def build_copies(spec, case, n_copies):
    """n_copies independent device copies of every weight tensor."""
    import torch
    keys = [k for k in case if k != "x"]
    copies = [dict(case)]
    for _ in range(n_copies - 1):
        c = {"x": case["x"]}
        for k in keys:
            c[k] = case[k].clone()
        copies.append(c)
    torch.cuda.synchronize()
    return copies


def time_layer(spec, copies, x, steps, warmup):
    """Mean µs per fused call over `steps` calls rotating weight copies,
    timed with HIP events on the launch stream, plus the distinct expert
    count of the step."""
    import torch
    import mixture_experts_decode_sigmoid_amd as moe
    T = x.shape[0]
    layers = [moe.Layer(spec, dict(c, x=x), max_rows=T) for c in copies]
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        layers[i % len(layers)].forward(x, out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        layers[i % len(layers)].forward(x, out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    errs = [l.read_error() for l in layers]
    if any(errs):
        raise RuntimeError(f"device error bits {errs}")
    ids, _ = layers[0].route(x)
    distinct = len(set(ids.cpu().view(-1).tolist()))
    return ms * 1000.0 / steps, distinct


def cpu_baseline(spec, case, budget_s=12.0):
    """The fp64 oracle on host cores, whole one-row layer, repeated up to
    about budget_s seconds."""
    import numpy as np
    import fixtures
    import oracle
    h0 = fixtures.host_case(case, experts=[])
    ids, _, _, _ = oracle.route(spec, h0["x"], h0["router_w"], h0["bias"])
    used = sorted(set(ids.ravel().tolist()))
    h = fixtures.host_case(case, experts=used)
    threads = oracle.max_threads()
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.forward(spec, h, nthreads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 5:
            break
    t = float(np.median(times))
    b_alg = fixtures.algorithmic_bytes(spec, len(used))
    return dict(value=round(b_alg / t / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
                sample=f"{HEADLINE}: whole one-row layer ({len(used)} routed + 1 shared expert), "
                       f"median of {len(times)} calls, {t:.3f} s per call")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (for PMC byte-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this layer is measured on a single MI355X; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import fixtures
    import mixture_experts_decode_sigmoid_amd as moe
    moe.lib()
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    spec, case = fixtures.make_workload(HEADLINE, device="cuda")
    copies = build_copies(spec, case, N_COPIES)
    us, distinct = time_layer(spec, copies, case["x"], args.steps, args.warmup)
    b_alg = fixtures.algorithmic_bytes(spec, distinct)
    gbs = b_alg / (us * 1e-6) / 1e9

    extra = {}
    if not args.no_extra:
        for name in EXTRA:
            sname, T, rows, seed, req = fixtures.WORKLOADS[name]
            # this workload's activations and router; expert weights are the
            # rotating copies above (same shapes and distribution)
            head = fixtures.make_case(spec, T, seed, device="cuda", rows=rows, requests=req, experts=False)
            cps = []
            for c in copies:
                c2 = dict(c)
                c2["router_w"] = head["router_w"]
                c2["bias"] = head["bias"]
                cps.append(c2)
            steps = max(20, args.steps // (4 if T > 8 else 2))
            us_t, d_t = time_layer(spec, cps, head["x"], steps, max(5, args.warmup // 2))
            b_t = fixtures.algorithmic_bytes(spec, d_t)
            extra[name] = dict(rows=T, distinct_experts=d_t, us_per_call=round(us_t, 2),
                               algorithmic_bytes=b_t, gbs=round(b_t / (us_t * 1e-6) / 1e9, 1),
                               frac_of_peak=round(b_t / (us_t * 1e-6) / 1e9 / PEAK_HBM_GBS, 4))

        del copies
        torch.cuda.empty_cache()
        for name in EXTRA_SHARD:
            spec_s, case_s = fixtures.make_workload(name, device="cuda")
            cps = build_copies(spec_s, case_s, N_COPIES)
            T = case_s["x"].shape[0]
            us_t, d_t = time_layer(spec_s, cps, case_s["x"], max(20, args.steps // 2), max(5, args.warmup // 2))
            b_t = fixtures.algorithmic_bytes(spec_s, d_t)
            extra[name] = dict(rows=T, distinct_experts=d_t, us_per_call=round(us_t, 2),
                               algorithmic_bytes=b_t, gbs=round(b_t / (us_t * 1e-6) / 1e9, 1),
                               frac_of_peak=round(b_t / (us_t * 1e-6) / 1e9 / PEAK_HBM_GBS, 4))
            del cps, case_s
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(spec, case)

    line = {
        "metric": "µs per fused MoE layer call & achieved HBM GB/s at 1/8/64 decode rows",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1000.0, 5),
        "us_per_call": round(us, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; weights ~N(0,0.02) quantised to FP8 E4M3 with 128x128 fp32 scales)",
        "config": {"workload": "DeepSeek-V3-shaped MoE layer, 1 decode row (hidden 7168, inter 2048, "
                               "256 experts top-8 in 8 groups keep 4, 1 shared)",
                   "rows": 1, "distinct_experts": distinct, "algorithmic_bytes": b_alg,
                   "weight_copies_rotated": N_COPIES},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic_from_profiles(HEADLINE)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
