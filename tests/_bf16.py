"""Brute-force bf16 round-to-nearest-even over the table of every finite bf16
value (torch's bf16 -> float64 cast, a library routine), for pins that must
not lean on the oracle's own rounding."""
from __future__ import annotations

import math

import numpy as np
import torch


def table():
    """All finite non-negative bf16 values, ascending, with their codes."""
    codes = np.arange(0, 0x7F80, dtype=np.uint16)
    vals = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return codes, vals


def brute_rne(v, codes, vals):
    """bf16 code of the float v, rounded to nearest, ties to even (None for NaN)."""
    if v != v:
        return None
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    top = vals[-1]
    half_over = top + (top - vals[-2]) / 2  # halfway to 2^128
    if a >= half_over:
        return sign | 0x7F80
    i = int(np.searchsorted(vals, a, side="right")) - 1  # vals[i] <= a
    if i == len(vals) - 1:
        return sign | int(codes[i])
    lo, hi = vals[i], vals[i + 1]
    if a - lo < hi - a:
        c = codes[i]
    elif a - lo > hi - a:
        c = codes[i + 1]
    else:
        c = codes[i] if codes[i] % 2 == 0 else codes[i + 1]
    return sign | int(c)
