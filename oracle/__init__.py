"""ctypes binding of the plain fp64 CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline
leg of the benchmark are the only callers.  The product path
(mixture_experts_decode_sigmoid_amd) never imports this package, and this
package never imports the product.  Arrays are host numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT_FP8_B128 = 0
FMT_MXFP4 = 1


def build() -> str:
    """Compile liboracle.so with gcc (fp64, OpenMP, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class Cfg(C.Structure):
    _fields_ = [("hidden", C.c_int), ("inter", C.c_int), ("shared_inter", C.c_int),
                ("n_experts", C.c_int), ("top_k", C.c_int), ("n_group", C.c_int),
                ("topk_group", C.c_int), ("n_shared", C.c_int),
                ("routed_scale", C.c_double), ("routed_fmt", C.c_int), ("bias_bf16", C.c_int),
                ("expert_first", C.c_int), ("expert_count", C.c_int)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB)
        P = C.c_void_p
        L.oracle_dec_bf16.argtypes = [C.c_uint16]; L.oracle_dec_bf16.restype = C.c_double
        L.oracle_dec_e4m3.argtypes = [C.c_uint8]; L.oracle_dec_e4m3.restype = C.c_double
        L.oracle_dec_e2m1.argtypes = [C.c_uint8]; L.oracle_dec_e2m1.restype = C.c_double
        L.oracle_dec_e8m0.argtypes = [C.c_uint8]; L.oracle_dec_e8m0.restype = C.c_double
        L.oracle_bf16_rne.argtypes = [C.c_double]; L.oracle_bf16_rne.restype = C.c_uint16
        L.oracle_weight.argtypes = [C.c_int, P, P, C.c_int, C.c_int, C.c_int, C.c_int]
        L.oracle_weight.restype = C.c_double
        L.oracle_scores.argtypes = [C.POINTER(Cfg), P, P, P, P, P, P]
        L.oracle_scores.restype = None
        L.oracle_route.argtypes = [C.POINTER(Cfg), P, C.c_int, P, P, P, P, P, P]
        L.oracle_route.restype = C.c_int
        L.oracle_groups.argtypes = [C.POINTER(Cfg), C.c_int, P, P, P, P, P, P, P]
        L.oracle_groups.restype = C.c_int
        L.oracle_expert_ffn.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, P, P, P, P]
        L.oracle_expert_ffn.restype = None
        L.oracle_forward_rows.argtypes = [C.POINTER(Cfg), P, C.c_int, P, C.c_int, P, P,
                                          P, P, P, P, P, P, P, P, P, P, C.c_int]
        L.oracle_forward_rows.restype = C.c_int
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = C.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else C.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def make_cfg(spec) -> Cfg:
    """spec: a mapping with the layer's sizes and routing parameters."""
    return Cfg(int(spec["hidden"]), int(spec["inter"]), int(spec["shared_inter"]),
               int(spec["n_experts"]), int(spec["top_k"]), int(spec["n_group"]),
               int(spec["topk_group"]), int(spec["n_shared"]), float(spec["routed_scale"]),
               int(spec["routed_fmt"]), int(spec["bias_bf16"]),
               int(spec.get("expert_first", 0)), int(spec.get("expert_count", 0)))


def dec_bf16(v): return lib().oracle_dec_bf16(int(v))
def dec_e4m3(v): return lib().oracle_dec_e4m3(int(v))
def dec_e2m1(v): return lib().oracle_dec_e2m1(int(v))
def dec_e8m0(v): return lib().oracle_dec_e8m0(int(v))
def bf16_rne(v): return lib().oracle_bf16_rne(float(v))


def weight(fmt, q, scale, N, K, n, k):
    return lib().oracle_weight(int(fmt), _p(q), _p(scale), int(N), int(K), int(n), int(k))


def scores(spec, x_row, router_w, bias):
    cfg = make_cfg(spec)
    E = cfg.n_experts
    x_row = _c(x_row, np.uint16); router_w = _c(router_w, np.uint16); bias = np.ascontiguousarray(bias)
    l = np.empty(E); s = np.empty(E); b = np.empty(E)
    lib().oracle_scores(C.byref(cfg), _p(x_row), _p(router_w), _p(bias), _p(l), _p(s), _p(b))
    return l, s, b


def route(spec, x, router_w, bias):
    """x: [T,H] uint16 (bf16 bits). Returns ids [T,K] int32, w [T,K] f64,
    gap_expert [T], gap_group [T]."""
    cfg = make_cfg(spec)
    x = _c(x, np.uint16); router_w = _c(router_w, np.uint16); bias = np.ascontiguousarray(bias)
    T = x.shape[0]
    K = cfg.top_k
    ids = np.empty((T, K), np.int32); w = np.empty((T, K)); ge = np.empty(T); gg = np.empty(T)
    rc = lib().oracle_route(C.byref(cfg), _p(x), T, _p(router_w), _p(bias), _p(ids), _p(w), _p(ge), _p(gg))
    if rc:
        raise ValueError(f"oracle_route rc={rc}")
    return ids, w, ge, gg


def groups(spec, ids):
    """Distinct-expert grouping. Returns (expert[G], ncols[G], col_start[G],
    cols[sum ncols] (= r*16+slot), use_group[T*K])."""
    cfg = make_cfg(spec)
    ids = _c(ids, np.int32)
    T = ids.shape[0]
    K = cfg.top_k
    gmax = 1 + T * K
    G = np.zeros(1, np.int32)
    ge = np.empty(gmax, np.int32); gn = np.empty(gmax, np.int32); gs = np.empty(gmax, np.int32)
    cols = np.empty(max(1, T * (K + 1)), np.int32); ug = np.empty(max(1, T * K), np.int32)
    rc = lib().oracle_groups(C.byref(cfg), T, _p(ids), _p(G), _p(ge), _p(gn), _p(gs), _p(cols), _p(ug))
    if rc:
        raise ValueError(f"oracle_groups rc={rc}")
    g = int(G[0])
    return ge[:g].copy(), gn[:g].copy(), gs[:g].copy(), cols[: int(gn[:g].sum())].copy(), ug[: T * K].copy()


def expert_ffn(fmt, H, Iexp, w_gate_up, s_gate_up, w_down, s_down, x64):
    w_gate_up = np.ascontiguousarray(w_gate_up); s_gate_up = np.ascontiguousarray(s_gate_up)
    w_down = np.ascontiguousarray(w_down); s_down = np.ascontiguousarray(s_down)
    x64 = _c(x64, np.float64)
    y = np.empty(H); mid = np.empty(Iexp)
    lib().oracle_expert_ffn(int(fmt), int(H), int(Iexp), _p(w_gate_up), _p(s_gate_up),
                            _p(w_down), _p(s_down), _p(x64), _p(y), _p(mid))
    return y, mid


def forward(spec, case, rows=None, nthreads=0):
    """Runs the layer on host arrays.

    case: mapping with numpy arrays x [T,H] u16, router_w [E,H] u16, bias,
    and per-expert lists (or [E,...] arrays) w_gate_up, s_gate_up, w_down,
    s_down (entries may be None for experts no row uses), and shared
    sh_w_gate_up, sh_s_gate_up, sh_w_down, sh_s_down.
    rows: optional list of rows to compute (others are left 0 / NaN).
    Returns (out64 [T,H] f64, out_bf16 [T,H] u16)."""
    cfg = make_cfg(spec)
    x = _c(case["x"], np.uint16)
    T, H = x.shape
    E = cfg.n_experts
    keep = []

    def ptrs(arrs):
        P = (C.c_void_p * E)()
        for e in range(E):
            a = arrs[e]
            if a is None:
                P[e] = None
            else:
                a = np.ascontiguousarray(a)
                keep.append(a)
                P[e] = a.ctypes.data
        return P

    pw = ptrs(case["w_gate_up"]); ps = ptrs(case["s_gate_up"])
    pd = ptrs(case["w_down"]); pds = ptrs(case["s_down"])
    rw = _c(case["router_w"], np.uint16); bias = np.ascontiguousarray(case["bias"])
    if cfg.n_shared:
        shw = np.ascontiguousarray(case["sh_w_gate_up"]); shs = _c(case["sh_s_gate_up"], np.float32)
        shd = np.ascontiguousarray(case["sh_w_down"]); shds = _c(case["sh_s_down"], np.float32)
    else:
        shw = shs = shd = shds = None
    if rows is None:
        rows = list(range(T))
    rows_a = np.asarray(rows, np.int32)
    out64 = np.full((T, H), np.nan)
    outb = np.zeros((T, H), np.uint16)
    rc = lib().oracle_forward_rows(C.byref(cfg), _p(x), T, _p(rows_a), len(rows_a), _p(rw), _p(bias),
                                   C.cast(pw, C.c_void_p), C.cast(ps, C.c_void_p),
                                   C.cast(pd, C.c_void_p), C.cast(pds, C.c_void_p),
                                   _p(shw), _p(shs), _p(shd), _p(shds), _p(out64), _p(outb), int(nthreads))
    if rc:
        raise ValueError(f"oracle_forward_rows rc={rc}")
    return out64, outb


def forward_residual(spec, case, residual, rows=None, nthreads=0):
    """The layer with the residual add folded in: the add that follows the
    routed and shared expert paths as the fourth launch of the unfused layout
    ("Daily AI Hotspot 2026-08-21: Shared-Expert Fusion Lands on NVIDIA and
    AMD the Same Day", section "Most Worth Your Attention Today").  Reading:
    out = bf16_RNE(layer + residual), the sum in fp64, rounded once.
    residual: [T,H] bf16 bits (u16).  Returns (out64, out_bf16) as forward
    does, for the listed rows."""
    out64, _ = forward(spec, case, rows=rows, nthreads=nthreads)
    res = _c(residual, np.uint16)
    T, H = res.shape
    o64 = np.full((T, H), np.nan)
    ob = np.zeros((T, H), np.uint16)
    for r in (range(T) if rows is None else rows):
        for h in range(H):
            v = float(out64[r, h]) + dec_bf16(res[r, h])
            o64[r, h] = v
            ob[r, h] = bf16_rne(v)
    return o64, ob


def max_threads() -> int:
    return int(lib().oracle_max_threads())
