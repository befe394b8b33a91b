"""The C-ABI library loads, exports every symbol include/moe.h declares, and
rejects bad arguments on the host before any launch (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

import fixtures
import mixture_experts_decode_sigmoid_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(moe_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    L = moe.lib()
    names = _declared()
    assert {"moe_route", "moe_forward", "moe_workspace_size", "moe_read_error", "moe_strerror"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(moe.EXPORTS)


def _cfg(**over):
    spec = fixtures.spec_with("v3")
    spec.update(over)
    return moe.make_config(spec, 8)


def test_workspace_size_and_config_checks():
    n = moe.moe_workspace_size(_cfg())
    assert n > 8 * 9 * 2048 * 2
    bad = [
        (dict(hidden=100), moe.MOE_ERR_SHAPE),
        (dict(inter=0), moe.MOE_ERR_SHAPE),
        (dict(top_k=9), moe.MOE_ERR_SHAPE),
        (dict(n_experts=300), moe.MOE_ERR_SHAPE),
        (dict(n_group=7), moe.MOE_ERR_SHAPE),          # 256 % 7 != 0
        (dict(topk_group=9), moe.MOE_ERR_SHAPE),
        (dict(routed_fmt=5), moe.MOE_ERR_FORMAT),
        (dict(bias_bf16=0, n_group=1, topk_group=1, top_k=8), None),
    ]
    for over, code in bad:
        cfg = _cfg(**over)
        if over.get("routed_fmt") == 5:
            cfg.routed_fmt = 5
        out = C.c_size_t(0)
        rc = moe.lib().moe_workspace_size(C.byref(cfg), C.byref(out))
        assert rc == (code or moe.MOE_OK), (over, rc)
    cfg = _cfg()
    cfg.max_rows = 65
    assert moe.lib().moe_workspace_size(C.byref(cfg), C.byref(C.c_size_t())) == moe.MOE_ERR_ROWS
    assert moe.lib().moe_workspace_size(None, C.byref(C.c_size_t())) == moe.MOE_ERR_NULL


def test_forward_argument_errors_without_launch():
    L = moe.lib()
    cfg = _cfg()
    w = moe.MoeWeights()
    x = C.c_void_p(0x1000)
    # NULL weights
    assert L.moe_forward(C.byref(cfg), C.byref(w), x, 1, C.c_void_p(0x2000), C.c_void_p(0x4000), 1 << 30, None) == moe.MOE_ERR_NULL
    w = moe.MoeWeights(*([0x10000] * 10))
    # misaligned x
    assert L.moe_forward(C.byref(cfg), C.byref(w), C.c_void_p(0x1001), 1, C.c_void_p(0x2000), C.c_void_p(0x4000), 1 << 30, None) == moe.MOE_ERR_ALIGN
    # rows beyond max_rows
    assert L.moe_forward(C.byref(cfg), C.byref(w), x, 9, C.c_void_p(0x2000), C.c_void_p(0x4000), 1 << 30, None) == moe.MOE_ERR_ROWS
    assert L.moe_forward(C.byref(cfg), C.byref(w), x, -1, C.c_void_p(0x2000), C.c_void_p(0x4000), 1 << 30, None) == moe.MOE_ERR_ROWS
    # workspace too small
    assert L.moe_forward(C.byref(cfg), C.byref(w), x, 1, C.c_void_p(0x2000), C.c_void_p(0x4000), 16, None) == moe.MOE_ERR_WORKSPACE
    # route: NULL outputs are checked after the common validation
    assert L.moe_route(C.byref(cfg), C.byref(w), x, 1, None, None, C.c_void_p(0x4000), 16, None) == moe.MOE_ERR_WORKSPACE
    for code in range(0, 10):
        assert isinstance(moe.strerror(code), str)
