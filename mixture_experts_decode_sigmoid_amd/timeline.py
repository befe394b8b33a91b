"""Per-phase timeline of the fused layer from its in-kernel stamps.

    python -m mixture_experts_decode_sigmoid_amd.timeline [--build] WORKLOAD [--calls N]

The library built with MOE_TIMELINE (libmoe_timeline.so, beside libmoe.so)
has thread 0 of every workgroup (and lane 0 of every wave for the per-wave
stamps) write s_memrealtime (100 MHz) at phase boundaries into 64 slots per
CU placed after the workspace.  This tool runs the workload with rotating
weight copies (--save keeps every stamp as a .npy array), and for every stamp prints the median and maximum over CUs
(medians over calls) in microseconds from the earliest CU start of the call.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_TL = os.path.join(HERE, "libmoe_timeline.so")

# stamp slot -> phase boundary (thread 0 unless noted)
NAMES = {
    0: "kernel start",
    1: "logits stored",
    2: "routing start",
    9: "row 0 scores in (its routing wave; above 8 rows: each routing CU's row)",
    60: "row 0 keys formed",
    14: "row 0 group stage done",
    56: "row 0 top-k threshold found",
    57: "row 0 top-k candidates in LDS",
    15: "row 0 top-k done",
    58: "row 0 weights formed",
    59: "routed up/gate tables ready",
    61: "above 8 rows: picks stored (routing CUs)",
    63: "above 8 rows: thread 0 has its picks",
    10: "all rows routed",
    3: "groups built",
    11: "tables written",
    62: "up/gate ring opened",
    13: "up/gate ring filled",
    4: "up/gate phase end (wave 0)",
    12: "flag raised",
    5: "meeting crossed",
    6: "down phase end (wave 0)",
    7: "combine end",
}
WAVE_NAMES = {0: "up/gate end", 1: "down start", 2: "down end"}


def build():
    from mixture_experts_decode_sigmoid_amd import build as b
    return b.build(verbose=False, out=LIB_TL, defines=("MOE_TIMELINE",))


def run(workload: str, calls: int, copies: int = 4, save: str | None = None):
    import torch
    sys.path.insert(0, ROOT)
    import fixtures
    import mixture_experts_decode_sigmoid_amd as moe
    moe.use_library(LIB_TL)
    moe.lib()
    spec, case = fixtures.make_workload(workload, device="cuda")
    keys = [k for k in case if k != "x"]
    cps = [case] + [dict({k: case[k].clone() for k in keys}, x=case["x"]) for _ in range(copies - 1)]
    T = case["x"].shape[0]
    extra = 1024 * 16 * 8
    layers = [moe.Layer(spec, c, max_rows=T, ws_extra=extra) for c in cps]
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty_like(case["x"])
    stamps = []
    for i in range(calls + 4):
        L = layers[i % len(layers)]
        L.ws[L.ws_bytes:].zero_()
        L.forward(case["x"], out)
        torch.cuda.synchronize()
        if i >= 4:
            tl = L.ws[L.ws_bytes:L.ws_bytes + ncu * 64 * 8].cpu().numpy().view(np.uint64).reshape(ncu, 64)
            stamps.append(tl.astype(np.int64))
        if L.read_error():
            raise RuntimeError("device error bits set")
    S = np.stack(stamps)                      # [calls, ncu, 64]
    t0 = S[:, :, 0].min(axis=1)[:, None]      # earliest start per call
    us = (S - t0[:, :, None]) / 100.0         # 100 MHz ticks -> us
    valid = S > 0
    if save:
        np.save(save, np.where(valid, us, np.nan))
    print(f"{workload}: {calls} calls, {ncu} CUs; median / max over CUs, median over calls (us)")
    rows = []
    for i, name in NAMES.items():
        if not valid[:, :, i].any():
            continue
        med = np.median([np.median(us[c, valid[c, :, i], i]) for c in range(len(S)) if valid[c, :, i].any()])
        mx = np.median([np.max(us[c, valid[c, :, i], i]) for c in range(len(S)) if valid[c, :, i].any()])
        rows.append((med, name, mx))
    for k, name in WAVE_NAMES.items():
        sl = [16 + 8 * k + w for w in range(8)]
        v = valid[:, :, sl]
        if not v.any():
            continue
        vals = us[:, :, sl]
        med = np.median([np.median(vals[c][v[c]]) for c in range(len(S)) if v[c].any()])
        mx = np.median([np.max(vals[c][v[c]]) for c in range(len(S)) if v[c].any()])
        rows.append((med, f"waves: {name}", mx))
    for med, name, mx in sorted(rows):
        print(f"  {name:40s} {med:8.2f} {mx:8.2f}")
    # per wave index: the median over CUs and calls of each per-wave stamp
    print("  per wave 0..7 (median over CUs and calls)")
    for k, name in WAVE_NAMES.items():
        sl = [16 + 8 * k + w for w in range(8)]
        if not valid[:, :, sl].any():
            continue
        vals = np.where(valid[:, :, sl], us[:, :, sl], np.nan)
        print(f"  {name:28s} " + " ".join(f"{np.nanmedian(vals[:, :, w]):7.2f}" for w in range(8)))
    # spread over CUs of the phase ends (median over calls of each percentile),
    # and by XCD (workgroup i runs on XCD i mod 8)
    print("  spread over CUs: p10 / p50 / p90 / max; then the median per XCD 0..7")
    for i in (11, 4, 12, 5, 6, 7):
        if not valid[:, :, i].any():
            continue
        v = np.where(valid[:, :, i], us[:, :, i], np.nan)
        q = np.nanmedian(np.nanpercentile(v, [10, 50, 90, 100], axis=1), axis=1)
        xcd = [np.nanmedian(v[:, x::8]) for x in range(8)]
        print(f"  {NAMES[i]:28s} " + " ".join(f"{v:7.2f}" for v in q) + "  |" +
              " ".join(f"{v:6.1f}" for v in xcd))
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("--calls", type=int, default=30)
    ap.add_argument("--build", action="store_true")
    ap.add_argument("--save", help="also write the stamps (calls x CUs x 64, us; NaN where unset) as .npy")
    a = ap.parse_args()
    if a.build:
        print(build())
    run(a.workload, a.calls, save=a.save)


if __name__ == "__main__":
    main()
