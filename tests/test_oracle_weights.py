"""Pins of the oracle's dequantised weight element (block-scale grid, nibble
order and E8M0 scale axis): a round trip through the seeded quantiser must
land within the format's rounding bound of the original fp32 weights.  A
transposed scale grid, a swapped nibble or a wrong scale axis moves most
elements far outside that bound (the blocks are given very different
magnitudes on purpose).
"""
import numpy as np
import torch

import fixtures


def _dequant_all(orc, fmt, q, s, N, K):
    return np.array([[orc.weight(fmt, q, s, N, K, n, k) for k in range(K)] for n in range(N)])


def test_fp8_block_round_trip(orc):
    g = torch.Generator().manual_seed(5)
    N, K = 256, 384
    w = torch.randn(N, K, generator=g) * 0.02
    # make every 128x128 block's magnitude different
    blk_gain = torch.tensor([[1.0, 40.0, 0.01], [7.0, 0.3, 250.0]])
    w = w * blk_gain.repeat_interleave(128, 0).repeat_interleave(128, 1)
    q, s = fixtures.quant_fp8_b128(w)
    q = q.numpy(); s = s.numpy()
    assert s.shape == (2, 3)
    deq = _dequant_all(orc, fixtures.FMT_FP8_B128, q, s, N, K)
    w64 = w.double().numpy()
    sb = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)
    bound = np.abs(w64) * 2.0 ** -4 + sb * 2.0 ** -10
    assert np.all(np.abs(deq - w64) <= bound)
    # the largest element of each block maps to +-448 * scale exactly
    for a in range(2):
        for b in range(3):
            blk = deq[a * 128:(a + 1) * 128, b * 128:(b + 1) * 128]
            assert np.max(np.abs(blk)) == 448.0 * float(s[a, b])


def test_mxfp4_round_trip(orc):
    g = torch.Generator().manual_seed(6)
    N, K = 8, 256
    w = torch.randn(N, K, generator=g) * 0.02
    w = w * (10.0 ** torch.arange(-2, 6, dtype=torch.float32).repeat_interleave(32))[None, :]
    q, s = fixtures.quant_mxfp4(w)
    q = q.numpy(); s = s.numpy()
    assert q.shape == (N, K // 2) and s.shape == (N, K // 32)
    deq = _dequant_all(orc, fixtures.FMT_MXFP4, q, s, N, K)
    w64 = w.double().numpy()
    X = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, 1)
    # grid values are multiples of 0.5*2^X below 2 and of 2^X above: a
    # rounding error is at most a quarter of the local step, 1 below 4 and
    # 2 between 4 and 6, and saturation at 6 loses at most 2 * 2^X
    err = np.abs(deq - w64)
    assert np.all(err <= 0.25 * np.abs(w64) + 0.25 * X + 1e-30)
    assert np.all(np.abs(deq) <= 6 * X)
    # every dequantised element is a grid point times its block scale
    grid = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    assert set(np.unique(np.abs(deq / X))) <= grid


def test_fp8_scale_is_multiplicative(orc):
    """Doubling one block scale doubles exactly that block's elements."""
    g = torch.Generator().manual_seed(7)
    w = torch.randn(256, 256, generator=g) * 0.02
    q, s = fixtures.quant_fp8_b128(w)
    q = q.numpy(); s = s.numpy()
    s2 = s.copy(); s2[1, 0] *= 2
    a = _dequant_all(orc, 0, q, s, 256, 256)
    b = _dequant_all(orc, 0, q, s2, 256, 256)
    assert np.array_equal(b[128:, :128], 2 * a[128:, :128])
    mask = np.ones_like(a, bool); mask[128:, :128] = False
    assert np.array_equal(a[mask], b[mask])
