"""Shared helpers of the GPU tests: seeded cases on the device, the oracle on
host copies of the experts a step uses, and the parity metrics."""
from __future__ import annotations

import sys

import numpy as np
import torch

import fixtures
import oracle
import mixture_experts_decode_sigmoid_amd as moe

REL_L2 = 2e-2
MAX_ABS = 1e-1


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).double().numpy()


def gpu_case(spec, T, seed, rows="iid", requests=1):
    return fixtures.make_case(spec, T, seed, device="cuda", rows=rows, requests=max(1, requests))


def host_router_case(case):
    return fixtures.host_case(case, experts=[])


def oracle_route(spec, case):
    h = host_router_case(case)
    return oracle.route(spec, h["x"], h["router_w"], h["bias"])


def oracle_rows(spec, case, rows, ids=None, nthreads=0):
    """Oracle output rows (fp64 and bf16 bits) for the listed rows, with host
    copies of only the experts those rows use."""
    if ids is None:
        ids, _, _, _ = oracle_route(spec, case)
    used = sorted(set(int(e) for r in rows for e in ids[r]))
    h = fixtures.host_case(case, experts=used, spec=spec)
    o64, ob = oracle.forward(spec, h, rows=list(rows), nthreads=nthreads)
    return o64, ob


def parity(gpu_bits: np.ndarray, o64: np.ndarray, rows):
    g = bf16_to_f64(gpu_bits[rows])
    r = o64[rows]
    rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    mx = float(np.max(np.abs(g - r)))
    return rel, mx


def run_forward(layer: moe.Layer, x: torch.Tensor, check: bool = True) -> np.ndarray:
    """One forward; with `check`, also asserts that the call raised no device
    error bit (a timed-out wait, a non-finite score or sum)."""
    out = layer.forward(x)
    torch.cuda.synchronize()
    if check:
        bits = layer.read_error()
        assert bits == 0, f"device error bits {bits:#x}"
    return fixtures.bits16(out)
