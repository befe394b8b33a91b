"""moe_forward_noalloc (the workspace in the library's static per-device
array) against moe_forward (a caller's workspace), through the C ABI: the
same kernel, so the outputs must be equal bit for bit.  Two calls in a row,
the second with a smaller batch, then another layer shape on the same
static array, then the first again."""
import numpy as np
import pytest
import torch

import fixtures
import mixture_experts_decode_sigmoid_amd as moe
from _gpu import gpu_case, say

pytestmark = pytest.mark.gpu

V3R = dict(hidden=1024, inter=256, shared_inter=256, n_experts=256, top_k=8, n_group=8, topk_group=4)
MX = dict(hidden=2048, inter=1536, shared_inter=512, n_experts=16, top_k=6, routed_fmt=1, bias_bf16=1)


def _both(layer, x):
    ref = layer.forward(x)
    got = torch.empty_like(x)
    moe.moe_forward_noalloc(layer.cfg, layer.w, x, got)
    torch.cuda.synchronize()
    assert layer.read_error() == 0
    return fixtures.bits16(ref), fixtures.bits16(got)


def test_noalloc_matches_forward():
    say("noalloc: V3 routing layer, 37 rows then 5")
    spec = fixtures.spec_with("tiny", **V3R)
    case = gpu_case(spec, 37, 91, rows="corr", requests=9)
    layer = moe.Layer(spec, case, max_rows=37)
    for T in (37, 5):
        ref, got = _both(layer, case["x"][:T].contiguous())
        assert np.array_equal(got, ref), T
    say("noalloc: MXFP4 layer, 16 rows then 1")
    spec2 = fixtures.spec_with("tiny", **MX)
    case2 = gpu_case(spec2, 16, 92, rows="corr", requests=4)
    layer2 = moe.Layer(spec2, case2, max_rows=16)
    for T in (16, 1):
        ref, got = _both(layer2, case2["x"][:T].contiguous())
        assert np.array_equal(got, ref), T
    say("noalloc: the first layer again, 8 rows")
    ref, got = _both(layer, case["x"][:8].contiguous())
    assert np.array_equal(got, ref)


def test_noalloc_argument_errors():
    spec = fixtures.spec_with("tiny")
    case = gpu_case(spec, 2, 93)
    layer = moe.Layer(spec, case, max_rows=2)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_noalloc(layer.cfg, layer.w, torch.zeros(3, 256, dtype=torch.bfloat16, device="cuda"),
                                torch.empty(3, 256, dtype=torch.bfloat16, device="cuda"))
    assert e.value.code == moe.MOE_ERR_ROWS
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_noalloc(layer.cfg, layer.w, case["x"], case["x"])
    assert e.value.code == moe.MOE_ERR_ALIAS
