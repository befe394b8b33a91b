"""The MXFP4 scale packer (moe_pack_mxfp4_scales) against the tiled layout
include/moe.h defines: byte j of row n's K-block kb at
((n/16)*(k/256) + kb)*128 + (n%16)*8 + j.  Byte work: bit-exact."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_decode_sigmoid_amd as moe

pytestmark = pytest.mark.gpu


def _tiled(src: np.ndarray, rows: int, k: int) -> np.ndarray:
    kb = k // 256
    return src.reshape(rows // 16, 16, kb, 8).transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("rows,k", [(16, 256), (48, 512), (4096, 7168), (3 * 2048, 2048)])
def test_pack_matches_the_tiled_layout(rows, k):
    g = torch.Generator().manual_seed(rows + k)
    src = torch.randint(0, 256, (rows * k // 32,), dtype=torch.uint8, generator=g)
    d_src = src.cuda()
    d_dst = torch.full_like(d_src, 0x5A)
    moe.moe_pack_mxfp4_scales(d_src, d_dst, rows, k)
    torch.cuda.synchronize()
    assert np.array_equal(d_dst.cpu().numpy(), _tiled(src.numpy(), rows, k))


def test_pack_argument_errors():
    L = moe.lib()
    a = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    b = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    P = moe._ptr
    assert L.moe_pack_mxfp4_scales(None, P(b), 16, 256, None) == moe.MOE_ERR_NULL
    assert L.moe_pack_mxfp4_scales(P(a), P(b), 8, 256, None) == moe.MOE_ERR_SHAPE
    assert L.moe_pack_mxfp4_scales(P(a), P(b), 16, 300, None) == moe.MOE_ERR_SHAPE
    assert L.moe_pack_mxfp4_scales(P(a), P(a), 16, 256, None) == moe.MOE_ERR_ALIAS
