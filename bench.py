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
weights and scales once, plus the router weights), B_alg / mean call time;
median and p90 of the per-call times are reported beside the mean.  The same
figures at 8 rows (2 requests x 4 MTP rows) and 64 independent rows, for the
tiny layer, the DeepSeek-V4-style MXFP4 top-6 layer at 16 rows and the
tensor-parallel shares are reported under "extra".  stream_read_gbs is what
a plain streaming-read kernel reaches on this GPU; every fraction of the
8 TB/s peak is also given as a fraction of it.  cpu_baseline times the fp64
oracle on the host's cores on the one-row layer; cpu_extra adds one-core
figures.
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
# workloads with weights of their own: the tiny layer, the V4-style MXFP4
# layer, and one GPU's share of the V3 layer under 8- and 4-way tensor
# parallelism and under 8-way expert parallelism
EXTRA_OWN = ("tiny_t1", "v4_t16", "v3tp8_t1", "v3tp8_t8", "v3tp4_t1", "v3tp4_t8", "v3ep8_t8", "v3ep8_t64")
STREAM_BYTES = 4 << 30
PREFILL_ROWS, PREFILL_CHUNK = 256, 64


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("moe_kernels.hip", "moe_api.cpp", "moe_internal.h"):
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


def note(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def time_layer(spec, copies, x, steps, warmup, unfused=False, marked=True):
    """Times `steps` fused calls (or calls of the unfused four-launch layout)
    rotating weight copies.  The mean comes from two HIP events on the launch
    stream around exactly `steps` back-to-back calls (whole-job time over
    steps).  With `marked`, a second pass of the same calls with an event
    after every call gives the per-call distribution; those markers add about
    3 us per call (measured), so its median and p90 sit above the mean.
    Returns (mean us, per-call us array or None, distinct held experts)."""
    import numpy as np
    import torch
    import fixtures
    import mixture_experts_decode_sigmoid_amd as moe
    T = x.shape[0]
    layers = [moe.Layer(spec, dict(c, x=x), max_rows=T) for c in copies]
    out = torch.empty_like(x)
    t_r, t_s = torch.empty_like(x), torch.empty_like(x)

    def call(l):
        if unfused:
            moe.moe_forward_unfused(l.cfg, l.w, x, out, t_r, t_s, l.ws)
        else:
            l.forward(x, out)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        call(layers[i % len(layers)])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        call(layers[i % len(layers)])
    b.record(stream)
    torch.cuda.synchronize()
    mean = a.elapsed_time(b) * 1000.0 / steps
    per = None
    if marked:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            call(layers[i % len(layers)])
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = np.array([ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(steps)])
    errs = [l.read_error() for l in layers]
    if any(errs):
        raise RuntimeError(f"device error bits {errs}")
    ids, _ = layers[0].route(x)
    distinct = fixtures.held_distinct(spec, ids.cpu().view(-1).tolist())
    return mean, per, distinct


def time_prefill(spec, copies, x, steps, warmup, stream_gbs):
    """Times moe_forward_prefill over all rows of x (chunks of PREFILL_CHUNK
    rows, one fused launch each) rotating weight copies, between two HIP
    events on the launch stream.  The algorithmic bytes are each chunk's own
    (its distinct experts' weights once, plus the router), summed."""
    import torch
    import fixtures
    import mixture_experts_decode_sigmoid_amd as moe
    T = x.shape[0]
    layers = [moe.Layer(spec, dict(c, x=x[:PREFILL_CHUNK]), max_rows=PREFILL_CHUNK) for c in copies]
    out = torch.empty_like(x)

    def call(l):
        moe.moe_forward_prefill(l.cfg, l.w, x, out, l.ws)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        call(layers[i % len(layers)])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        call(layers[i % len(layers)])
    b.record(stream)
    torch.cuda.synchronize()
    mean = a.elapsed_time(b) * 1000.0 / steps
    errs = [l.read_error() for l in layers]
    if any(errs):
        raise RuntimeError(f"device error bits {errs}")
    b_alg, distinct = 0, []
    for r0 in range(0, T, PREFILL_CHUNK):
        ids, _ = layers[0].route(x[r0:r0 + PREFILL_CHUNK].contiguous())
        d = fixtures.held_distinct(spec, ids.cpu().view(-1).tolist())
        distinct.append(d)
        b_alg += fixtures.algorithmic_bytes(spec, d)
    gbs = b_alg / (mean * 1e-6) / 1e9
    return dict(rows=T, chunk_rows=PREFILL_CHUNK, launches=len(distinct), distinct_experts_per_chunk=distinct,
                us_per_call=round(mean, 2), us_per_row=round(mean / T, 2), algorithmic_bytes=b_alg,
                gbs=round(gbs, 1), frac_of_peak=round(gbs / PEAK_HBM_GBS, 4),
                frac_of_stream_read=round(gbs / stream_gbs, 4) if stream_gbs else None, steps=steps)


def summary(mean, per, b_alg, stream_gbs):
    import numpy as np
    gbs = b_alg / (mean * 1e-6) / 1e9
    d = dict(us_per_call=round(mean, 2))
    if per is not None:
        d.update(us_median_marked=round(float(np.median(per)), 2), us_p90_marked=round(float(np.percentile(per, 90)), 2))
    d.update(algorithmic_bytes=b_alg, gbs=round(gbs, 1), frac_of_peak=round(gbs / PEAK_HBM_GBS, 4))
    if stream_gbs:
        d["frac_of_stream_read"] = round(gbs / stream_gbs, 4)
    return d


def stream_read_gbs(reps=10):
    """GB/s of a plain streaming read of a 4 GiB buffer (the library's probe
    kernel), best grid of a small sweep, median of `reps` timed reads."""
    import numpy as np
    import torch
    import mixture_experts_decode_sigmoid_amd as moe
    buf = torch.ones(STREAM_BYTES // 4, dtype=torch.int32, device="cuda")
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    best = 0.0
    for mult in (4, 8, 16):
        blocks = ncu * mult
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        for _ in range(2):
            moe.moe_probe_stream_read(buf, sink, blocks)
        times = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            moe.moe_probe_stream_read(buf, sink, blocks)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        best = max(best, STREAM_BYTES / float(np.median(times)) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return round(best, 1)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_time(spec, case, rows, threads, budget_s, max_runs=5):
    """Median seconds of the oracle over `rows` (host copies of only the
    experts they use), and how many runs it took."""
    import numpy as np
    import fixtures
    import oracle
    h0 = fixtures.host_case(case, experts=[])
    ids, _, _, _ = oracle.route(spec, h0["x"], h0["router_w"], h0["bias"])
    used = sorted(set(int(e) for r in rows for e in ids[r]))
    h = fixtures.host_case(case, experts=used)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.forward(spec, h, rows=list(rows), nthreads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= max_runs:
            break
    d_all = len(set(ids.ravel().tolist()))
    return float(np.median(times)), len(times), d_all


def cpu_baseline(spec, case, budget_s=12.0):
    """The fp64 oracle on host cores, whole one-row layer, repeated up to
    about budget_s seconds."""
    import fixtures
    import oracle
    threads = oracle.max_threads()
    t, n, d = _oracle_time(spec, case, [0], threads, budget_s)
    b_alg = fixtures.algorithmic_bytes(spec, d)
    return dict(value=round(b_alg / t / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
                sample=f"{HEADLINE}: whole one-row layer ({d} routed + 1 shared expert), "
                       f"median of {n} calls, {t:.3f} s per call", cpu_model=cpu_model())


def cpu_extra(spec, case, device):
    """One-core oracle figures: the tiny layer (1 row), the V3 layer at 1 row
    and at 8 rows (2 of the 8 rows timed, scaled to the call)."""
    import fixtures
    res = {}
    spec_t, case_t = fixtures.make_workload("tiny_t1", device=device)
    t, n, d = _oracle_time(spec_t, case_t, [0], 1, 2.0)
    res["tiny_t1"] = dict(cores=1, s_per_call=round(t, 6), runs=n,
                          gbs=round(fixtures.algorithmic_bytes(spec_t, d) / t / 1e9, 4))
    t, n, d = _oracle_time(spec, case, [0], 1, 4.0, max_runs=1)
    res["v3_t1"] = dict(cores=1, s_per_call=round(t, 3), runs=n,
                        gbs=round(fixtures.algorithmic_bytes(spec, d) / t / 1e9, 4))
    sname, T, rows, seed, req = fixtures.WORKLOADS["v3_t8"]
    head = fixtures.make_case(spec, T, seed, device=device, rows=rows, requests=req, experts=False)
    c8 = dict(case, x=head["x"], router_w=head["router_w"], bias=head["bias"])
    t, n, d = _oracle_time(spec, c8, [0, 5], 1, 8.0, max_runs=1)
    t_call = t * T / 2
    res["v3_t8"] = dict(cores=1, s_per_call=round(t_call, 3), runs=n, sample="rows 0 and 5 timed, scaled by 8/2",
                        gbs=round(fixtures.algorithmic_bytes(spec, d) / t_call / 1e9, 4))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--workload", default=HEADLINE,
                    help="time this workload only (for profiling runs; implies --no-extra --no-cpu)")
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

    if args.workload != HEADLINE:
        spec, case = fixtures.make_workload(args.workload, device="cuda")
        copies = build_copies(spec, case, N_COPIES)
        mean, per, distinct = time_layer(spec, copies, case["x"], args.steps, args.warmup)
        d = summary(mean, per, fixtures.algorithmic_bytes(spec, distinct), None)
        print(json.dumps(dict(workload=args.workload, rows=case["x"].shape[0], distinct_experts=distinct, **d)),
              flush=True)
        return

    stream_gbs = stream_read_gbs()
    note(f"stream read {stream_gbs} GB/s")

    spec, case = fixtures.make_workload(HEADLINE, device="cuda")
    copies = build_copies(spec, case, N_COPIES)
    us, per, distinct = time_layer(spec, copies, case["x"], args.steps, args.warmup)
    b_alg = fixtures.algorithmic_bytes(spec, distinct)
    gbs = b_alg / (us * 1e-6) / 1e9
    head = summary(us, per, b_alg, stream_gbs)
    note(f"{HEADLINE}: {us:.2f} us")

    extra = {}
    if not args.no_extra:
        for name in EXTRA:
            sname, T, rows, seed, req = fixtures.WORKLOADS[name]
            # this workload's activations and router; expert weights are the
            # rotating copies above (same shapes and distribution)
            hd = fixtures.make_case(spec, T, seed, device="cuda", rows=rows, requests=req, experts=False)
            cps = []
            for c in copies:
                c2 = dict(c)
                c2["router_w"] = hd["router_w"]
                c2["bias"] = hd["bias"]
                cps.append(c2)
            steps = max(20, args.steps // (4 if T > 8 else 2))
            m_t, per_t, d_t = time_layer(spec, cps, hd["x"], steps, max(5, args.warmup // 2))
            extra[name] = dict(rows=T, distinct_experts=d_t,
                               **summary(m_t, per_t, fixtures.algorithmic_bytes(spec, d_t), stream_gbs))
            note(f"{name}: {extra[name]['us_per_call']} us")

        # fusion A/B: the fused pass against the unfused four-launch layout
        # (routed MoE, shared gate/up, shared down, add), alternating rounds
        ab = {}
        for name in (HEADLINE,) + EXTRA:
            sname, T, rows, seed, req = fixtures.WORKLOADS[name]
            hd = fixtures.make_case(spec, T, seed, device="cuda", rows=rows, requests=req, experts=False)
            cps = [dict(c, router_w=hd["router_w"], bias=hd["bias"]) for c in copies]
            steps = max(20, args.steps // (4 if T > 8 else 2))
            f_us, u_us = [], []
            for _ in range(3):
                m_f, _, _ = time_layer(spec, cps, hd["x"], steps, 5, marked=False)
                m_u, _, _ = time_layer(spec, cps, hd["x"], steps, 5, unfused=True, marked=False)
                f_us.append(m_f)
                u_us.append(m_u)
            f, u = min(f_us), min(u_us)
            ab[name] = dict(rows=T, fused_us=round(f, 2), unfused_us=round(u, 2),
                            fusion_gain_pct=round(100.0 * (u - f) / u, 2), rounds=3, statistic="best of 3 means")
            note(f"fusion A/B {name}: fused {f:.2f} us, unfused {u:.2f} us")
        extra["fusion_ab"] = ab

        # the larger-T path: 256 independent rows through moe_forward_prefill
        # (consecutive fused calls of 64 rows, each its own launch)
        hd = fixtures.make_case(spec, PREFILL_ROWS, 5, device="cuda", rows="iid", requests=PREFILL_ROWS,
                                experts=False)
        cps = [dict(c, router_w=hd["router_w"], bias=hd["bias"]) for c in copies]
        extra["v3_prefill_t256"] = time_prefill(spec, cps, hd["x"], max(10, args.steps // 20), 3, stream_gbs)
        note(f"v3_prefill_t256: {extra['v3_prefill_t256']['us_per_call']} us")

        del copies
        torch.cuda.empty_cache()
        for name in EXTRA_OWN:
            spec_s, case_s = fixtures.make_workload(name, device="cuda")
            cps = build_copies(spec_s, case_s, N_COPIES)
            T = case_s["x"].shape[0]
            m_t, per_t, d_t = time_layer(spec_s, cps, case_s["x"], max(20, args.steps // 2), max(5, args.warmup // 2))
            extra[name] = dict(rows=T, distinct_experts=d_t,
                               **summary(m_t, per_t, fixtures.algorithmic_bytes(spec_s, d_t), stream_gbs))
            note(f"{name}: {extra[name]['us_per_call']} us")
            del cps, case_s
            torch.cuda.empty_cache()

    cpu = None
    cpu_x = None
    if not args.no_cpu:
        cpu = cpu_baseline(spec, case)
        note("cpu baseline done")
        if not args.no_extra:
            cpu_x = cpu_extra(spec, case, "cuda")

    line = {
        "metric": "µs per fused MoE layer call & achieved HBM GB/s at 1/8/64 decode rows",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1000.0, 5),
        "us_per_call": round(us, 2),
        "us_median_marked": head["us_median_marked"],
        "us_p90_marked": head["us_p90_marked"],
        "timing": "mean: two HIP events on the launch stream around the timed calls; "
                  "*_marked: a second pass with an event after every call (the markers add about 3 us per call)",
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
        "cpu_extra": cpu_x,
        "stream_read_gbs": stream_gbs,
        "frac_of_stream_read": round(gbs / stream_gbs, 4),
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
